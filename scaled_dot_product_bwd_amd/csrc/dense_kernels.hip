// dense_kernels.hip -- the three gfx950 kernels of the dense attention backward.
//
//   k_row_stats  query-block-major, once per row: m, l = sum exp(s - m) and
//                delta = rowsum(P * dP), the latter as dY . O with O = P V
//                accumulated online (equal in exact arithmetic).  The
//                statistics triple is the one ruDNN ordered_kernel.rs
//                `history_backward` consumes (max, denominator, delta).
//   k_kv_bwd     KV-block-major: per 128-key block, over its visible 32-query
//                chunks in ascending order, recompute S and P, then
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
// All five contractions run on 32x32 MFMA tiles (device_common.hpp).
#include "device_common.hpp"
#include "launch.hpp"

namespace attn {

// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void k_row_stats(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ RowTile<T, 32, D> Ks;
  __shared__ typename CReuseSrc<T, 32, D>::tile Vs;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = nb - 1 - (L % nb);  // the heaviest causal blocks first
  const int h = (L / nb) % p.H, b = L / (nb * p.H);
  const int i0 = blk * 128, iw = i0 + 32 * w, qi = iw + l32;
  const bool qvalid = qi < p.Sq;

  const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
  typename M::frag qf[NSD];
#pragma unroll
  for (int s = 0; s < NSD; ++s) qf[s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);

  const T *kbase = (const T *)p.k + b * p.ks[0] + h * p.ks[2];
  const T *vbase = (const T *)p.v + b * p.vs[0] + h * p.vs[2];
  const int ilast = min(i0 + 128, p.Sq) - 1;
  const int jlo = max(0, i0 + p.lo_off);
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x16{};

  for (int j0 = jlo & ~31; j0 <= jhi; j0 += 32) {
    __syncthreads();
    stage_rows<T, D>(kbase, p.ks[1], j0, p.Sk, Ks);
    if constexpr (sizeof(T) == 2)
      stage_cols<D>(vbase, p.vs[1], j0, p.Sk, Vs);  // V only transposed (A of O^T = V^T P^T)
    else
      stage_rows<T, D>(vbase, p.vs[1], j0, p.Sk, Vs);
    __syncthreads();
    if (MODE == MODE_INDEX && tile_none_visible(p, iw, j0)) continue;
    const bool check = MODE != MODE_INDEX || !tile_all_visible(p, iw, j0);

    // S^T = K Q^T: rows = keys (A from LDS), columns = this lane's query.
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NSD; ++s) sacc = M::mma(Ks.frag(l32, s, half), qf[s], sacc);

    float sc[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = masked_score<MODE>(p, sacc[r], b, h, qi, j0 + kr(r, half), check);
      mloc = fmaxf(mloc, sc[r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = fast_exp2(sc[r] - m_use);
      psum += sc[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] *= alpha;

    // O^T += V^T P^T: A = V^T from LDS, B = P straight from the S^T tile.
#pragma unroll
    for (int st = 0; st < M::CSTEPS; ++st) {
      const typename M::frag pf = creuse<T>(sc, st);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        o[t] = M::mma(CReuseSrc<T, 32, D>::frag(Vs, 32 * t + l32, st, half), pf, o[t]);
    }
  }

  // delta = dY . O / l  (O^T tile: lane holds its query, d = 32 t + kr(r, half)).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
  float dsum = 0.f;
  if (qvalid) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t + 8 * g + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum += (float)grow[d0 + e] * o[t][4 * g + e];
      }
  }
  dsum += __shfl_xor(dsum, 32);
  if (qvalid && half == 0) {
    const int64_t row = ((int64_t)b * p.H + h) * p.Sq + qi;
    const bool empty = !(l_tot > 0.f);
    p.st_m[row] = empty ? -INFINITY : m_run * kLn2;
    p.st_l[row] = empty ? 0.f : l_tot;
    p.st_delta[row] = empty ? 0.f : dsum / l_tot;
    p.st_lse2[row] = empty ? INFINITY : m_run + __log2f(l_tot);
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void k_kv_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ RowTile<T, 32, D> Qs, Gs;
  __shared__ TTile<32, (sizeof(T) == 2 ? D : 1)> Qt, Gt;  // bf16 only
  __shared__ __attribute__((aligned(16))) float lse_s[32];
  __shared__ __attribute__((aligned(16))) float del_s[32];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = L % nb;  // key block 0 sees the most queries under a causal mask
  const int h = (L / nb) % p.H, b = L / (nb * p.H);
  const int j0b = blk * 128, jw = j0b + 32 * w, kj = jw + l32;
  const bool kvalid = kj < p.Sk;

  const T *krow = (const T *)p.k + b * p.ks[0] + (int64_t)(kvalid ? kj : 0) * p.ks[1] + h * p.ks[2];
  const T *vrow = (const T *)p.v + b * p.vs[0] + (int64_t)(kvalid ? kj : 0) * p.vs[1] + h * p.vs[2];
  typename M::frag kf[NSD], vf[NSD];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    kf[s] = load_frag<T>(krow, s * KS + half * KL, kvalid);
    vf[s] = load_frag<T>(vrow, s * KS + half * KL, kvalid);
  }

  const T *qbase = (const T *)p.q + b * p.qs[0] + h * p.qs[2];
  const T *gbase = (const T *)p.dy + b * p.dys[0] + h * p.dys[2];
  const int64_t srow0 = ((int64_t)b * p.H + h) * p.Sq;
  const int jlast = min(j0b + 128, p.Sk) - 1;
  const int ilo = max(0, (int)max((int64_t)j0b - p.hi_off, (int64_t)0));
  const int ihi = min(p.Sq - 1, (int)min((int64_t)jlast - p.lo_off, (int64_t)kBig));

  f32x16 dk[NT], dv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dk[t] = dv[t] = f32x16{};

  for (int i0 = ilo & ~31; i0 <= ihi; i0 += 32) {
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
      stage_rows<T, D>(qbase, p.qs[1], i0, p.Sq, Qs, &Qt);
      stage_rows<T, D>(gbase, p.dys[1], i0, p.Sq, Gs, &Gt);
    } else {
      stage_rows<T, D>(qbase, p.qs[1], i0, p.Sq, Qs);
      stage_rows<T, D>(gbase, p.dys[1], i0, p.Sq, Gs);
    }
    if (tid < 32) {
      const bool valid = i0 + tid < p.Sq;
      lse_s[tid] = valid ? p.st_lse2[srow0 + i0 + tid] : INFINITY;
      del_s[tid] = valid ? p.st_delta[srow0 + i0 + tid] : 0.f;
    }
    __syncthreads();
    if (MODE == MODE_INDEX && tile_none_visible(p, i0, jw)) continue;
    const bool check = MODE != MODE_INDEX || !tile_all_visible(p, i0, jw);

    // S = Q K^T and dP = dY V^T: rows = queries (A from LDS), columns = this lane's key.
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      sacc = M::mma(Qs.frag(l32, s, half), kf[s], sacc);
      pacc = M::mma(Gs.frag(l32, s, half), vf[s], pacc);
    }
    float pv[16], dsv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&lse_s[8 * g + 4 * half]);
      const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&del_s[8 * g + 4 * half]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float s2 = masked_score<MODE>(p, sacc[r], b, h, i0 + kr(r, half), kj, check);
        const float pr = fast_exp2(s2 - lse4[e]);
        pv[r] = pr;
        dsv[r] = pr * (pacc[r] - del4[e]) * p.scale;
      }
    }
    // dV^T += dY^T P and dK^T += Q^T dS: A = transposed rows from LDS, B = C reuse.
#pragma unroll
    for (int st = 0; st < M::CSTEPS; ++st) {
      const typename M::frag pf = creuse<T>(pv, st);
      const typename M::frag sf = creuse<T>(dsv, st);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (sizeof(T) == 2) {
          dv[t] = M::mma(Gt.frag(32 * t + l32, st, half), pf, dv[t]);
          dk[t] = M::mma(Qt.frag(32 * t + l32, st, half), sf, dk[t]);
        } else {
          dv[t] = M::mma(CReuseSrc<T, 32, D>::frag(Gs, 32 * t + l32, st, half), pf, dv[t]);
          dk[t] = M::mma(CReuseSrc<T, 32, D>::frag(Qs, 32 * t + l32, st, half), sf, dk[t]);
        }
      }
    }
  }

  if (!kvalid) return;
  T *dkrow = (T *)p.dk + b * p.dks[0] + (int64_t)kj * p.dks[1] + h * p.dks[2];
  T *dvrow = (T *)p.dv + b * p.dvs[0] + (int64_t)kj * p.dvs[1] + h * p.dvs[2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * t + 8 * g + 4 * half;
      if (p.need_dk)
        store4<T>(dkrow + d0, dk[t][4 * g], dk[t][4 * g + 1], dk[t][4 * g + 2], dk[t][4 * g + 3]);
      if (p.need_dv)
        store4<T>(dvrow + d0, dv[t][4 * g], dv[t][4 * g + 1], dv[t][4 * g + 2], dv[t][4 * g + 3]);
    }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void k_dq_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ RowTile<T, 32, D> Ks, Vs;
  __shared__ TTile<32, (sizeof(T) == 2 ? D : 1)> Kt;  // bf16 only

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = nb - 1 - (L % nb);
  const int h = (L / nb) % p.H, b = L / (nb * p.H);
  const int i0 = blk * 128, iw = i0 + 32 * w, qi = iw + l32;
  const bool qvalid = qi < p.Sq;

  const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
  const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
  typename M::frag qf[NSD], gf[NSD];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    qf[s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);
    gf[s] = load_frag<T>(grow, s * KS + half * KL, qvalid);
  }
  const int64_t srow = ((int64_t)b * p.H + h) * p.Sq + (qvalid ? qi : 0);
  const float lse = qvalid ? p.st_lse2[srow] : INFINITY;
  const float del = qvalid ? p.st_delta[srow] : 0.f;

  const T *kbase = (const T *)p.k + b * p.ks[0] + h * p.ks[2];
  const T *vbase = (const T *)p.v + b * p.vs[0] + h * p.vs[2];
  const int ilast = min(i0 + 128, p.Sq) - 1;
  const int jlo = max(0, i0 + p.lo_off);
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));

  f32x16 dq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dq[t] = f32x16{};

  for (int j0 = jlo & ~31; j0 <= jhi; j0 += 32) {
    __syncthreads();
    if constexpr (sizeof(T) == 2)
      stage_rows<T, D>(kbase, p.ks[1], j0, p.Sk, Ks, &Kt);
    else
      stage_rows<T, D>(kbase, p.ks[1], j0, p.Sk, Ks);
    stage_rows<T, D>(vbase, p.vs[1], j0, p.Sk, Vs);
    __syncthreads();
    if (MODE == MODE_INDEX && tile_none_visible(p, iw, j0)) continue;
    const bool check = MODE != MODE_INDEX || !tile_all_visible(p, iw, j0);

    // S^T = K Q^T and dP^T = V dY^T: rows = keys, columns = this lane's query.
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      sacc = M::mma(Ks.frag(l32, s, half), qf[s], sacc);
      pacc = M::mma(Vs.frag(l32, s, half), gf[s], pacc);
    }
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float s2 = masked_score<MODE>(p, sacc[r], b, h, qi, j0 + kr(r, half), check);
      const float pr = fast_exp2(s2 - lse);
      dsv[r] = pr * (pacc[r] - del) * p.scale;
    }
    // dQ^T += K^T dS^T: A = K^T from LDS, B = dS straight from the tile.
#pragma unroll
    for (int st = 0; st < M::CSTEPS; ++st) {
      const typename M::frag sf = creuse<T>(dsv, st);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (sizeof(T) == 2)
          dq[t] = M::mma(Kt.frag(32 * t + l32, st, half), sf, dq[t]);
        else
          dq[t] = M::mma(CReuseSrc<T, 32, D>::frag(Ks, 32 * t + l32, st, half), sf, dq[t]);
      }
    }
  }

  if (!qvalid) return;
  T *dqrow = (T *)p.dq + b * p.dqs[0] + (int64_t)qi * p.dqs[1] + h * p.dqs[2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4<T>(dqrow + 32 * t + 8 * g + 4 * half, dq[t][4 * g], dq[t][4 * g + 1], dq[t][4 * g + 2],
                dq[t][4 * g + 3]);
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
