/*
 * attn_oracle.c -- plain, slow CPU reference ("the oracle") for the scaled
 * dot-product attention backward pass, computed in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library
 * never calls it.
 *
 * Sources (web pages, cited by title and the function on the page):
 *   [rlx-cpu]  docs.rs rlx-cpu 0.2.17, source page src/attention_bwd.rs
 *   [rlx-wgpu] docs.rs rlx-wgpu 0.2.1, source page src/kernels/attention_bwd.wgsl
 *   [rlx-metal] docs.rs rlx-metal 0.2.12, source page src/attention_bwd_gpu.rs
 *   [ruDNN]    docs.rs ruDNN 0.1.43, source page src/paged_attention/ordered_kernel.rs
 *
 * Every result here is the plain definition written out: full Sq x Sk score,
 * probability and gradient matrices per (batch, head), no tiling, no online
 * softmax, no reordering beyond what the definition states.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *   - masked scores are EXCLUDED from the softmax (an exact -inf), rather than
 *     set to a finite sentinel; for any row with a visible key the two agree
 *     exactly in float64;
 *   - a row with no visible key has P = 0, m = -inf, l = 0, delta = 0 and
 *     contributes nothing (as [ruDNN] `history_backward` skips rows whose
 *     denominator is zero);
 *   - the causal rule may be combined with key padding or bias through
 *     `causal_flag`, applied after them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Mask kinds: the numeric codes the pages use for MaskKind
 * ([rlx-wgpu] `mask_score`, [rlx-metal] `use_gpu`). */
enum {
  ORC_MASK_NONE = 0,
  ORC_MASK_CAUSAL = 1,
  ORC_MASK_KEYPAD = 2, /* "Custom": per-key validity compared to a threshold */
  ORC_MASK_WINDOW = 3, /* SlidingWindow(w) */
  ORC_MASK_BIAS = 4    /* additive bias */
};

typedef struct {
  int64_t B, H, Sq, Sk, D;
  const double *q, *k, *v, *dy; /* [B,S,H,D], contiguous */
  int mask_kind;
  int causal_flag;
  int64_t window;
  const double *mask;  /* keypad validity or additive bias */
  int64_t mst[4];      /* element strides of `mask` over (b, h, q, k) */
  double thr;          /* keypad: key hidden iff mask value < thr */
  double scale;
  double *dq, *dk, *dv;           /* [B,S,H,D] outputs, each may be NULL */
  double *m, *l, *delta, *delta_o; /* [B,H,Sq] row statistics, may be NULL */
  double *out;                    /* forward output O = P V, [B,Sq,H,D], may be NULL */
  int64_t next_head;              /* work counter shared by threads */
  pthread_mutex_t lock;
} dense_job;

/* One (b, h) head, straight from the definition.
 * Scores:   [rlx-cpu] `backward_dense_head_all` (S = scale * Q K^T).
 * Masks:    [rlx-cpu] `backward_dense_head_all` (custom then bias) and
 *           `apply_synthetic_mask` (causal / sliding window, offset Sk - Sq
 *           saturating at 0).
 * Softmax:  plain max-subtracted row softmax ([rlx-wgpu] `softmax_row`).
 * Backward: dV = P^T dY; dP = dY V^T; dS = P (dP - rowsum(P dP)) scale;
 *           dQ = dS K; dK = dS^T Q ([rlx-cpu] `backward_dense_head_all`). */
static void dense_head(dense_job *J, int64_t b, int64_t h, double *S,
                       unsigned char *vis, double *P, double *dP, double *dS,
                       double *orow) {
  const int64_t Sq = J->Sq, Sk = J->Sk, D = J->D;
  const int64_t rs = J->H * D; /* distance between consecutive rows of one head */
  const double *Q = J->q + b * Sq * rs + h * D;
  const double *dY = J->dy + b * Sq * rs + h * D;
  const double *K = J->k + b * Sk * rs + h * D;
  const double *V = J->v + b * Sk * rs + h * D;
  const int kind = J->mask_kind;
  const int causal = kind == ORC_MASK_CAUSAL ||
                     ((kind == ORC_MASK_KEYPAD || kind == ORC_MASK_BIAS) && J->causal_flag);
  /* Query row i sits at absolute position q_off + i (saturating Sk - Sq). */
  const int64_t q_off = Sk > Sq ? Sk - Sq : 0;

  for (int64_t i = 0; i < Sq; ++i) {
    const int64_t abs_q = q_off + i;
    for (int64_t j = 0; j < Sk; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += Q[i * rs + d] * K[j * rs + d];
      double s = J->scale * acc;
      int visible = 1;
      const double *mv = J->mask ? J->mask + b * J->mst[0] + h * J->mst[1] +
                                       i * J->mst[2] + j * J->mst[3]
                                 : NULL;
      if (kind == ORC_MASK_KEYPAD && *mv < J->thr) visible = 0;
      if (kind == ORC_MASK_BIAS) s += *mv; /* added after the scale, unscaled */
      if (causal && j > abs_q) visible = 0;
      if (kind == ORC_MASK_WINDOW) {
        const int64_t lo = abs_q >= J->window ? abs_q - J->window : 0;
        if (j < lo || j > abs_q) visible = 0;
      }
      S[i * Sk + j] = s;
      vis[i * Sk + j] = (unsigned char)visible;
    }
  }

  /* Row softmax over the visible keys. */
  for (int64_t i = 0; i < Sq; ++i) {
    double mx = -INFINITY;
    int any = 0;
    for (int64_t j = 0; j < Sk; ++j)
      if (vis[i * Sk + j]) {
        any = 1;
        if (S[i * Sk + j] > mx) mx = S[i * Sk + j];
      }
    double den = 0.0;
    if (any)
      for (int64_t j = 0; j < Sk; ++j)
        if (vis[i * Sk + j]) den += exp(S[i * Sk + j] - mx);
    for (int64_t j = 0; j < Sk; ++j)
      P[i * Sk + j] = (any && vis[i * Sk + j]) ? exp(S[i * Sk + j] - mx) / den : 0.0;
    if (J->m) J->m[(b * J->H + h) * Sq + i] = any ? mx : -INFINITY;
    if (J->l) J->l[(b * J->H + h) * Sq + i] = den;
  }

  /* dP = dY V^T */
  for (int64_t i = 0; i < Sq; ++i)
    for (int64_t j = 0; j < Sk; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += dY[i * rs + d] * V[j * rs + d];
      dP[i * Sk + j] = acc;
    }

  /* delta_i = rowsum(P * dP); dS = P (dP - delta) scale.
   * The same delta also equals dY_i . O_i with O = P V; it is computed
   * separately so that a test can compare the two. */
  for (int64_t i = 0; i < Sq; ++i) {
    double delta = 0.0;
    for (int64_t j = 0; j < Sk; ++j) delta += P[i * Sk + j] * dP[i * Sk + j];
    for (int64_t j = 0; j < Sk; ++j)
      dS[i * Sk + j] = P[i * Sk + j] * (dP[i * Sk + j] - delta) * J->scale;
    if (J->delta) J->delta[(b * J->H + h) * Sq + i] = delta;
    /* O_i = sum_j P_ij V_j, accumulated in ascending j for every d. */
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    for (int64_t j = 0; j < Sk; ++j)
      for (int64_t d = 0; d < D; ++d) orow[d] += P[i * Sk + j] * V[j * rs + d];
    double dyo = 0.0;
    for (int64_t d = 0; d < D; ++d) dyo += dY[i * rs + d] * orow[d];
    if (J->delta_o) J->delta_o[(b * J->H + h) * Sq + i] = dyo;
    if (J->out)
      for (int64_t d = 0; d < D; ++d) J->out[b * Sq * rs + i * rs + h * D + d] = orow[d];
  }

  /* dV_j = sum_i P_ij dY_i and dK_j = sum_i dS_ij Q_i, in ascending i. */
  double *gV = J->dv ? J->dv + b * Sk * rs + h * D : NULL;
  double *gK = J->dk ? J->dk + b * Sk * rs + h * D : NULL;
  for (int64_t j = 0; j < Sk; ++j)
    for (int64_t d = 0; d < D; ++d) {
      if (gV) gV[j * rs + d] = 0.0;
      if (gK) gK[j * rs + d] = 0.0;
    }
  for (int64_t i = 0; i < Sq; ++i)
    for (int64_t j = 0; j < Sk; ++j)
      for (int64_t d = 0; d < D; ++d) {
        if (gV) gV[j * rs + d] += P[i * Sk + j] * dY[i * rs + d];
        if (gK) gK[j * rs + d] += dS[i * Sk + j] * Q[i * rs + d];
      }
  /* dQ_i = sum_j dS_ij K_j, in ascending j. */
  if (J->dq) {
    double *gQ = J->dq + b * Sq * rs + h * D;
    for (int64_t i = 0; i < Sq; ++i) {
      for (int64_t d = 0; d < D; ++d) gQ[i * rs + d] = 0.0;
      for (int64_t j = 0; j < Sk; ++j)
        for (int64_t d = 0; d < D; ++d) gQ[i * rs + d] += dS[i * Sk + j] * K[j * rs + d];
    }
  }
}

static void *dense_worker(void *arg) {
  dense_job *J = (dense_job *)arg;
  const int64_t ss = J->Sq * J->Sk > 0 ? J->Sq * J->Sk : 1;
  double *S = (double *)malloc(sizeof(double) * ss);
  double *P = (double *)malloc(sizeof(double) * ss);
  double *dP = (double *)malloc(sizeof(double) * ss);
  double *dS = (double *)malloc(sizeof(double) * ss);
  unsigned char *vis = (unsigned char *)malloc(ss);
  double *orow = (double *)malloc(sizeof(double) * J->D);
  if (S && P && dP && dS && vis && orow) {
    for (;;) {
      pthread_mutex_lock(&J->lock);
      const int64_t idx = J->next_head++;
      pthread_mutex_unlock(&J->lock);
      if (idx >= J->B * J->H) break;
      dense_head(J, idx / J->H, idx % J->H, S, vis, P, dP, dS, orow);
    }
  }
  free(S);
  free(P);
  free(dP);
  free(dS);
  free(vis);
  free(orow);
  return NULL;
}

/* Dense backward for all (b, h) heads.  Returns 0 on success, -1 on invalid
 * arguments.  Outputs that are NULL are not computed into.  Empty Sq or Sk
 * give zero gradients (and -inf / 0 statistics for rows with no keys). */
int oracle_attn_bwd(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                    const double *q, const double *k, const double *v, const double *dy,
                    int mask_kind, int causal_flag, int64_t window, const double *mask,
                    const int64_t *mask_strides, double threshold, double scale,
                    double *dq, double *dk, double *dv, double *row_m, double *row_l,
                    double *row_delta, double *row_delta_o, double *out, int nthreads) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return -1;
  if (mask_kind < ORC_MASK_NONE || mask_kind > ORC_MASK_BIAS) return -1;
  if (mask_kind == ORC_MASK_WINDOW && window < 0) return -1;
  if ((mask_kind == ORC_MASK_KEYPAD || mask_kind == ORC_MASK_BIAS) && (!mask || !mask_strides))
    return -1;
  const int64_t rs = H * D;
  /* Zero first: covers Sq == 0 or Sk == 0, where no head loop writes. */
  if (dq) memset(dq, 0, sizeof(double) * B * Sq * rs);
  if (dk) memset(dk, 0, sizeof(double) * B * Sk * rs);
  if (dv) memset(dv, 0, sizeof(double) * B * Sk * rs);
  if (out) memset(out, 0, sizeof(double) * B * Sq * rs);
  for (int64_t r = 0; r < B * H * Sq; ++r) {
    if (row_m) row_m[r] = -INFINITY;
    if (row_l) row_l[r] = 0.0;
    if (row_delta) row_delta[r] = 0.0;
    if (row_delta_o) row_delta_o[r] = 0.0;
  }
  if (B == 0 || H == 0 || Sq == 0 || Sk == 0) return 0;

  dense_job J;
  memset(&J, 0, sizeof J);
  J.B = B; J.H = H; J.Sq = Sq; J.Sk = Sk; J.D = D;
  J.q = q; J.k = k; J.v = v; J.dy = dy;
  J.mask_kind = mask_kind; J.causal_flag = causal_flag; J.window = window;
  J.mask = (mask_kind == ORC_MASK_KEYPAD || mask_kind == ORC_MASK_BIAS) ? mask : NULL;
  if (J.mask) memcpy(J.mst, mask_strides, sizeof J.mst);
  J.thr = threshold; J.scale = scale;
  J.dq = dq; J.dk = dk; J.dv = dv;
  J.m = row_m; J.l = row_l; J.delta = row_delta; J.delta_o = row_delta_o; J.out = out;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > B * H) nthreads = (int)(B * H);
  /* The calling thread works too; helpers that fail to start are skipped. */
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  int started = 0;
  for (int t = 1; t < nthreads; ++t)
    if (th && pthread_create(&th[started], NULL, dense_worker, &J) == 0) ++started;
  dense_worker(&J);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Paged, grouped-query history backward ([ruDNN] `history_backward`).
 *
 * Layouts (the page's own):
 *   q, dy       [nq, heads, D]              query rows packed across sequences
 *   k/v pools   [pool_pages * page_size, kv_heads, D]
 *   stats       [nq, heads, 3] = (max, denominator, delta)
 *   block_table [nseq, max_pages]            logical page -> physical page
 * Query head h reads KV head h / (heads / kv_heads).  Sequence s, logical
 * token t lives in physical slot block_table[s][t / page_size] * page_size +
 * t % page_size.  A row r of sequence s sees token t iff t < len_s and, when
 * causal, t <= pos_r.  Rows whose denominator is zero contribute nothing.
 * The listed pages are the physical pages of the logical pages
 * 0 .. ceil(len_s / page_size) - 1 of every sequence: each of their slots is
 * overwritten, with the gradient or with zero where no row sees it; every other
 * slot of the output pools keeps what the caller put there. */
static int paged_check(int nseq, const int32_t *seq_lens, const int32_t *block_table,
                       int max_pages, int nq, const int32_t *query_seq, int heads,
                       int kv_heads, int page_size, int pool_pages) {
  if (nseq < 0 || nq < 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads) return -1;
  if (page_size <= 0 || pool_pages < 0 || max_pages < 0) return -1;
  for (int s = 0; s < nseq; ++s) {
    if (seq_lens[s] < 0) return -1;
    const int np = (seq_lens[s] + page_size - 1) / page_size;
    if (np > max_pages) return -1;
    for (int p = 0; p < np; ++p) {
      const int phys = block_table[(int64_t)s * max_pages + p];
      if (phys < 0 || phys >= pool_pages) return -1;
    }
  }
  for (int r = 0; r < nq; ++r)
    if (query_seq[r] < 0 || query_seq[r] >= nseq) return -1;
  return 0;
}

typedef struct {
  int nseq, max_pages, nq, heads, kv_heads, D, page_size, pool_pages, causal;
  const int32_t *seq_lens, *block_table, *query_seq, *query_pos;
  double scale;
  const double *q, *dy, *k_pool, *v_pool, *stats_in;
  double *stats_out;  /* row statistics (paged_row_stats) */
  double *gk, *gv;    /* gradient accumulators over the whole pool (paged_kv_bwd) */
  /* latent variant: position width, position parts of queries and keys, and the
   * position-key gradient accumulator */
  int P;
  const double *qp, *kp_pool;
  double *gkp;
  int64_t next, count; /* work counter shared by threads */
  pthread_mutex_t lock;
} paged_job;

static int64_t paged_take(paged_job *J) {
  pthread_mutex_lock(&J->lock);
  const int64_t i = J->next++;
  pthread_mutex_unlock(&J->lock);
  return i < J->count ? i : -1;
}

static int64_t paged_slot(const paged_job *J, int s, int t) {
  return (int64_t)J->block_table[(int64_t)s * J->max_pages + t / J->page_size] * J->page_size +
         t % J->page_size;
}

/* Runs `worker` on `nthreads` threads (the caller included). */
static void paged_parallel(paged_job *J, void *(*worker)(void *), int nthreads) {
  pthread_mutex_init(&J->lock, NULL);
  J->next = 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > J->count) nthreads = J->count > 0 ? (int)J->count : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  int started = 0;
  for (int t = 1; t < nthreads; ++t)
    if (th && pthread_create(&th[started], NULL, worker, J) == 0) ++started;
  worker(J);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J->lock);
}

/* One query row r, every head: its visible scores, their softmax, and
 * delta = sum_t P dP, straight from the definition. */
static void *paged_stats_worker(void *arg) {
  paged_job *J = (paged_job *)arg;
  const int D = J->D, group = J->heads / J->kv_heads;
  int maxlen = 1;
  for (int s = 0; s < J->nseq; ++s)
    if (J->seq_lens[s] > maxlen) maxlen = J->seq_lens[s];
  double *sc = (double *)malloc(sizeof(double) * maxlen);
  double *dp = (double *)malloc(sizeof(double) * maxlen);
  unsigned char *vis = (unsigned char *)malloc(maxlen);
  for (int64_t r; sc && dp && vis && (r = paged_take(J)) >= 0;) {
    const int s = J->query_seq[r];
    const int len = J->seq_lens[s];
    for (int h = 0; h < J->heads; ++h) {
      const int g = h / group;
      const double *qr = J->q + (r * J->heads + h) * D;
      const double *gr = J->dy + (r * J->heads + h) * D;
      double mx = -INFINITY;
      int any = 0;
      for (int t = 0; t < len; ++t) {
        const int64_t slot = paged_slot(J, s, t);
        const double *kr = J->k_pool + (slot * J->kv_heads + g) * D;
        const double *vr = J->v_pool + (slot * J->kv_heads + g) * D;
        double a = 0.0, c = 0.0;
        for (int d = 0; d < D; ++d) { a += qr[d] * kr[d]; c += gr[d] * vr[d]; }
        sc[t] = J->scale * a;
        dp[t] = c;
        vis[t] = (unsigned char)(!J->causal || t <= J->query_pos[r]);
        if (vis[t]) { any = 1; if (sc[t] > mx) mx = sc[t]; }
      }
      double den = 0.0, delta = 0.0;
      if (any) {
        for (int t = 0; t < len; ++t) if (vis[t]) den += exp(sc[t] - mx);
        for (int t = 0; t < len; ++t) if (vis[t]) delta += exp(sc[t] - mx) / den * dp[t];
      }
      double *st = J->stats_out + (r * J->heads + h) * 3;
      st[0] = any ? mx : -INFINITY;
      st[1] = den;
      st[2] = delta;
    }
  }
  free(sc); free(dp); free(vis);
  return NULL;
}

/* Row statistics (max, denominator, delta) for the paged layout, from the
 * definition: the row's visible scores, their softmax, and delta = sum_t P dP.
 * [ruDNN] takes these as an input that a query-side kernel produces per row.
 * Rows are independent; threads split them. */
int oracle_paged_row_stats(int nseq, const int32_t *seq_lens, const int32_t *block_table,
                           int max_pages, int nq, const int32_t *query_seq,
                           const int32_t *query_pos, int heads, int kv_heads, int D,
                           int page_size, int pool_pages, int causal, double scale,
                           const double *q, const double *dy, const double *k_pool,
                           const double *v_pool, double *stats, int nthreads) {
  if (paged_check(nseq, seq_lens, block_table, max_pages, nq, query_seq, heads, kv_heads,
                  page_size, pool_pages))
    return -1;
  paged_job J;
  memset(&J, 0, sizeof J);
  J.nseq = nseq; J.max_pages = max_pages; J.nq = nq; J.heads = heads; J.kv_heads = kv_heads;
  J.D = D; J.page_size = page_size; J.pool_pages = pool_pages; J.causal = causal;
  J.seq_lens = seq_lens; J.block_table = block_table; J.query_seq = query_seq;
  J.query_pos = query_pos; J.scale = scale;
  J.q = q; J.dy = dy; J.k_pool = k_pool; J.v_pool = v_pool; J.stats_out = stats;
  J.count = nq;
  paged_parallel(&J, paged_stats_worker, nthreads);
  return 0;
}

/* dQ of one query row r, every head, from the supplied statistics: the
 * definition dQ_r = sum_t dS_rt K_t over the row's visible tokens, with
 * dS = P (dP - delta) scale and P = exp(s - max) / den; a zero denominator
 * gives a zero row (as [ruDNN] skips such rows). */
static void *paged_dq_worker(void *arg) {
  paged_job *J = (paged_job *)arg;
  const int D = J->D, group = J->heads / J->kv_heads;
  for (int64_t r; (r = paged_take(J)) >= 0;) {
    const int s = J->query_seq[r];
    const int len = J->seq_lens[s];
    for (int h = 0; h < J->heads; ++h) {
      const int g = h / group;
      const double *st = J->stats_in + (r * J->heads + h) * 3;
      const double *qr = J->q + (r * J->heads + h) * D;
      const double *gr = J->dy + (r * J->heads + h) * D;
      double *out = J->gk + (r * J->heads + h) * D;
      for (int d = 0; d < D; ++d) out[d] = 0.0;
      if (st[1] == 0.0) continue;
      for (int t = 0; t < len; ++t) {
        if (J->causal && t > J->query_pos[r]) continue;
        const int64_t slot = paged_slot(J, s, t);
        const double *kr = J->k_pool + (slot * J->kv_heads + g) * D;
        const double *vr = J->v_pool + (slot * J->kv_heads + g) * D;
        double a = 0.0, c = 0.0;
        for (int d = 0; d < D; ++d) { a += qr[d] * kr[d]; c += gr[d] * vr[d]; }
        const double p = exp(J->scale * a - st[0]) / st[1];
        const double ds = p * (c - st[2]) * J->scale;
        for (int d = 0; d < D; ++d) out[d] += ds * kr[d];
      }
    }
  }
  return NULL;
}

/* dQ [nq, heads, D] of the paged layout from supplied statistics (the query
 * side of [ruDNN] `history_backward`'s data).  Rows are independent; threads
 * split them. */
int oracle_paged_dq(int nseq, const int32_t *seq_lens, const int32_t *block_table, int max_pages,
                    int nq, const int32_t *query_seq, const int32_t *query_pos, int heads,
                    int kv_heads, int D, int page_size, int pool_pages, int causal, double scale,
                    const double *q, const double *dy, const double *k_pool, const double *v_pool,
                    const double *stats, double *dq, int nthreads) {
  if (paged_check(nseq, seq_lens, block_table, max_pages, nq, query_seq, heads, kv_heads,
                  page_size, pool_pages))
    return -1;
  paged_job J;
  memset(&J, 0, sizeof J);
  J.nseq = nseq; J.max_pages = max_pages; J.nq = nq; J.heads = heads; J.kv_heads = kv_heads;
  J.D = D; J.page_size = page_size; J.pool_pages = pool_pages; J.causal = causal;
  J.seq_lens = seq_lens; J.block_table = block_table; J.query_seq = query_seq;
  J.query_pos = query_pos; J.scale = scale;
  J.q = q; J.dy = dy; J.k_pool = k_pool; J.v_pool = v_pool; J.stats_in = stats;
  J.gk = dq;
  J.count = nq;
  paged_parallel(&J, paged_dq_worker, nthreads);
  return 0;
}

/* All contributions to the slots of one KV head g, in a fixed order:
 * sequences, then tokens, then query rows, then the group's heads. */
static void *paged_kv_worker(void *arg) {
  paged_job *J = (paged_job *)arg;
  const int D = J->D, group = J->heads / J->kv_heads;
  for (int64_t g; (g = paged_take(J)) >= 0;) {
    for (int s = 0; s < J->nseq; ++s) {
      const int len = J->seq_lens[s];
      for (int t = 0; t < len; ++t) {
        const int64_t slot = paged_slot(J, s, t);
        for (int r = 0; r < J->nq; ++r) {
          if (J->query_seq[r] != s) continue;
          if (J->causal && t > J->query_pos[r]) continue;
          for (int h = (int)g * group; h < ((int)g + 1) * group; ++h) {
            const double *st = J->stats_in + ((int64_t)r * J->heads + h) * 3;
            if (st[1] == 0.0) continue;
            const double *qr = J->q + ((int64_t)r * J->heads + h) * D;
            const double *gr = J->dy + ((int64_t)r * J->heads + h) * D;
            const double *kr = J->k_pool + (slot * J->kv_heads + g) * D;
            const double *vr = J->v_pool + (slot * J->kv_heads + g) * D;
            double a = 0.0, c = 0.0;
            for (int d = 0; d < D; ++d) { a += qr[d] * kr[d]; c += gr[d] * vr[d]; }
            const double p = exp(J->scale * a - st[0]) / st[1];
            const double ds = p * (c - st[2]) * J->scale;
            double *ak = J->gk + (slot * J->kv_heads + g) * D;
            double *av = J->gv + (slot * J->kv_heads + g) * D;
            for (int d = 0; d < D; ++d) { ak[d] += ds * qr[d]; av[d] += p * gr[d]; }
          }
        }
      }
    }
  }
  return NULL;
}

/* dK / dV into the page pools.  `dk_pool` / `dv_pool` hold the caller's pool
 * contents on entry (either may be NULL: not requested); on return every slot of
 * every listed page holds its gradient (zero where no row sees it) and every
 * other slot is unchanged.  KV heads have disjoint outputs; threads split them. */
int oracle_paged_kv_bwd(int nseq, const int32_t *seq_lens, const int32_t *block_table,
                        int max_pages, int nq, const int32_t *query_seq,
                        const int32_t *query_pos, int heads, int kv_heads, int D,
                        int page_size, int pool_pages, int causal, double scale,
                        const double *q, const double *dy, const double *k_pool,
                        const double *v_pool, const double *stats, double *dk_pool,
                        double *dv_pool, int nthreads) {
  if (paged_check(nseq, seq_lens, block_table, max_pages, nq, query_seq, heads, kv_heads,
                  page_size, pool_pages))
    return -1;
  const int64_t nslot = (int64_t)pool_pages * page_size;
  double *gk = (double *)calloc((size_t)(nslot * kv_heads * D) + 1, sizeof(double));
  double *gv = (double *)calloc((size_t)(nslot * kv_heads * D) + 1, sizeof(double));
  unsigned char *listed = (unsigned char *)calloc((size_t)pool_pages + 1, 1);
  if (!gk || !gv || !listed) { free(gk); free(gv); free(listed); return -1; }

  for (int s = 0; s < nseq; ++s) {
    const int np = (seq_lens[s] + page_size - 1) / page_size;
    for (int p = 0; p < np; ++p) listed[block_table[(int64_t)s * max_pages + p]] = 1;
  }
  paged_job J;
  memset(&J, 0, sizeof J);
  J.nseq = nseq; J.max_pages = max_pages; J.nq = nq; J.heads = heads; J.kv_heads = kv_heads;
  J.D = D; J.page_size = page_size; J.pool_pages = pool_pages; J.causal = causal;
  J.seq_lens = seq_lens; J.block_table = block_table; J.query_seq = query_seq;
  J.query_pos = query_pos; J.scale = scale;
  J.q = q; J.dy = dy; J.k_pool = k_pool; J.v_pool = v_pool; J.stats_in = stats;
  J.gk = gk; J.gv = gv;
  J.count = kv_heads;
  paged_parallel(&J, paged_kv_worker, nthreads);

  for (int pg = 0; pg < pool_pages; ++pg) {
    if (!listed[pg]) continue;
    const int64_t base = (int64_t)pg * page_size * kv_heads * D;
    const int64_t n = (int64_t)page_size * kv_heads * D;
    if (dk_pool) memcpy(dk_pool + base, gk + base, sizeof(double) * n);
    if (dv_pool) memcpy(dv_pool + base, gv + base, sizeof(double) * n);
  }
  free(gk); free(gv); free(listed);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Latent (MLA) variant of the paged history backward ([ruDNN]
 * `history_backward` with its `mla` switch on).  Every pool slot holds one
 * latent row c (width D) that is BOTH the key and the value, plus a position
 * key kp (width P).  A query row carries q (width D, in the latent space) and
 * qp (width P); dY has the latent width D.  Per visible (row, head, token):
 *   s  = scale (q . c + qp . kp)          the score uses both parts
 *   dP = dY . c                           the value is the latent itself
 *   p  = exp(s - max) / den,  ds = p (dP - delta) scale
 *   dc  += ds q + p dY                    the latent's key and value derivatives
 *   dkp += ds qp
 * There is no separate value gradient.  Reading: the value width equals the
 * latent width (dY rows are indexed with it while the latent's derivative runs
 * over the key width), and the value is the latent row. */

/* One query row r, every head: visible latent-variant scores, their softmax and
 * delta = sum_t P dP, from the definition. */
static void *paged_mla_stats_worker(void *arg) {
  paged_job *J = (paged_job *)arg;
  const int D = J->D, P = J->P, group = J->heads / J->kv_heads;
  int maxlen = 1;
  for (int s = 0; s < J->nseq; ++s)
    if (J->seq_lens[s] > maxlen) maxlen = J->seq_lens[s];
  double *sc = (double *)malloc(sizeof(double) * maxlen);
  double *dp = (double *)malloc(sizeof(double) * maxlen);
  unsigned char *vis = (unsigned char *)malloc(maxlen);
  for (int64_t r; sc && dp && vis && (r = paged_take(J)) >= 0;) {
    const int s = J->query_seq[r];
    const int len = J->seq_lens[s];
    for (int h = 0; h < J->heads; ++h) {
      const int g = h / group;
      const double *qr = J->q + (r * J->heads + h) * D;
      const double *qpr = J->qp + (r * J->heads + h) * P;
      const double *gr = J->dy + (r * J->heads + h) * D;
      double mx = -INFINITY;
      int any = 0;
      for (int t = 0; t < len; ++t) {
        const int64_t slot = paged_slot(J, s, t);
        const double *cr = J->k_pool + (slot * J->kv_heads + g) * D;
        const double *pr = J->kp_pool + (slot * J->kv_heads + g) * P;
        double a = 0.0, c = 0.0;
        for (int d = 0; d < D; ++d) { a += qr[d] * cr[d]; c += gr[d] * cr[d]; }
        for (int d = 0; d < P; ++d) a += qpr[d] * pr[d];
        sc[t] = J->scale * a;
        dp[t] = c;
        vis[t] = (unsigned char)(!J->causal || t <= J->query_pos[r]);
        if (vis[t]) { any = 1; if (sc[t] > mx) mx = sc[t]; }
      }
      double den = 0.0, delta = 0.0;
      if (any) {
        for (int t = 0; t < len; ++t) if (vis[t]) den += exp(sc[t] - mx);
        for (int t = 0; t < len; ++t) if (vis[t]) delta += exp(sc[t] - mx) / den * dp[t];
      }
      double *st = J->stats_out + (r * J->heads + h) * 3;
      st[0] = any ? mx : -INFINITY;
      st[1] = den;
      st[2] = delta;
    }
  }
  free(sc); free(dp); free(vis);
  return NULL;
}

/* (max, denominator, delta) per (row, head) of the latent variant. */
int oracle_paged_mla_row_stats(int nseq, const int32_t *seq_lens, const int32_t *block_table,
                               int max_pages, int nq, const int32_t *query_seq,
                               const int32_t *query_pos, int heads, int kv_heads, int D, int P,
                               int page_size, int pool_pages, int causal, double scale,
                               const double *q, const double *qp, const double *dy,
                               const double *latent_pool, const double *kp_pool, double *stats,
                               int nthreads) {
  if (P < 0 || paged_check(nseq, seq_lens, block_table, max_pages, nq, query_seq, heads,
                           kv_heads, page_size, pool_pages))
    return -1;
  paged_job J;
  memset(&J, 0, sizeof J);
  J.nseq = nseq; J.max_pages = max_pages; J.nq = nq; J.heads = heads; J.kv_heads = kv_heads;
  J.D = D; J.P = P; J.page_size = page_size; J.pool_pages = pool_pages; J.causal = causal;
  J.seq_lens = seq_lens; J.block_table = block_table; J.query_seq = query_seq;
  J.query_pos = query_pos; J.scale = scale;
  J.q = q; J.qp = qp; J.dy = dy; J.k_pool = latent_pool; J.kp_pool = kp_pool;
  J.stats_out = stats;
  J.count = nq;
  paged_parallel(&J, paged_mla_stats_worker, nthreads);
  return 0;
}

/* All latent-variant contributions to the slots of one KV head g, in a fixed
 * order: sequences, tokens, query rows, the group's heads. */
static void *paged_mla_kv_worker(void *arg) {
  paged_job *J = (paged_job *)arg;
  const int D = J->D, P = J->P, group = J->heads / J->kv_heads;
  for (int64_t g; (g = paged_take(J)) >= 0;) {
    for (int s = 0; s < J->nseq; ++s) {
      const int len = J->seq_lens[s];
      for (int t = 0; t < len; ++t) {
        const int64_t slot = paged_slot(J, s, t);
        const double *cr = J->k_pool + (slot * J->kv_heads + g) * D;
        const double *pr = J->kp_pool + (slot * J->kv_heads + g) * P;
        double *ac = J->gk + (slot * J->kv_heads + g) * D;
        double *ap = J->gkp + (slot * J->kv_heads + g) * P;
        for (int r = 0; r < J->nq; ++r) {
          if (J->query_seq[r] != s) continue;
          if (J->causal && t > J->query_pos[r]) continue;
          for (int h = (int)g * group; h < ((int)g + 1) * group; ++h) {
            const double *st = J->stats_in + ((int64_t)r * J->heads + h) * 3;
            if (st[1] == 0.0) continue;
            const double *qr = J->q + ((int64_t)r * J->heads + h) * D;
            const double *qpr = J->qp + ((int64_t)r * J->heads + h) * P;
            const double *gr = J->dy + ((int64_t)r * J->heads + h) * D;
            double a = 0.0, c = 0.0;
            for (int d = 0; d < D; ++d) { a += qr[d] * cr[d]; c += gr[d] * cr[d]; }
            for (int d = 0; d < P; ++d) a += qpr[d] * pr[d];
            const double p = exp(J->scale * a - st[0]) / st[1];
            const double ds = p * (c - st[2]) * J->scale;
            for (int d = 0; d < D; ++d) ac[d] += ds * qr[d] + p * gr[d];
            for (int d = 0; d < P; ++d) ap[d] += ds * qpr[d];
          }
        }
      }
    }
  }
  return NULL;
}

/* Latent and position-key gradients into their pools.  `dlat_pool` [slots,
 * kv_heads, D] and `dkp_pool` [slots, kv_heads, P] hold the caller's contents on
 * entry (either may be NULL: not requested); on return every slot of every
 * listed page holds its gradient (zero where no row sees it) and every other
 * slot is unchanged.  KV heads have disjoint outputs; threads split them. */
int oracle_paged_mla_kv_bwd(int nseq, const int32_t *seq_lens, const int32_t *block_table,
                            int max_pages, int nq, const int32_t *query_seq,
                            const int32_t *query_pos, int heads, int kv_heads, int D, int P,
                            int page_size, int pool_pages, int causal, double scale,
                            const double *q, const double *qp, const double *dy,
                            const double *latent_pool, const double *kp_pool,
                            const double *stats, double *dlat_pool, double *dkp_pool,
                            int nthreads) {
  if (P < 0 || paged_check(nseq, seq_lens, block_table, max_pages, nq, query_seq, heads,
                           kv_heads, page_size, pool_pages))
    return -1;
  const int64_t nslot = (int64_t)pool_pages * page_size;
  double *gc = (double *)calloc((size_t)(nslot * kv_heads * D) + 1, sizeof(double));
  double *gp = (double *)calloc((size_t)(nslot * kv_heads * P) + 1, sizeof(double));
  unsigned char *listed = (unsigned char *)calloc((size_t)pool_pages + 1, 1);
  if (!gc || !gp || !listed) { free(gc); free(gp); free(listed); return -1; }

  for (int s = 0; s < nseq; ++s) {
    const int np = (seq_lens[s] + page_size - 1) / page_size;
    for (int p = 0; p < np; ++p) listed[block_table[(int64_t)s * max_pages + p]] = 1;
  }
  paged_job J;
  memset(&J, 0, sizeof J);
  J.nseq = nseq; J.max_pages = max_pages; J.nq = nq; J.heads = heads; J.kv_heads = kv_heads;
  J.D = D; J.P = P; J.page_size = page_size; J.pool_pages = pool_pages; J.causal = causal;
  J.seq_lens = seq_lens; J.block_table = block_table; J.query_seq = query_seq;
  J.query_pos = query_pos; J.scale = scale;
  J.q = q; J.qp = qp; J.dy = dy; J.k_pool = latent_pool; J.kp_pool = kp_pool;
  J.stats_in = stats;
  J.gk = gc; J.gkp = gp;
  J.count = kv_heads;
  paged_parallel(&J, paged_mla_kv_worker, nthreads);

  for (int pg = 0; pg < pool_pages; ++pg) {
    if (!listed[pg]) continue;
    const int64_t nc = (int64_t)page_size * kv_heads * D, npp = (int64_t)page_size * kv_heads * P;
    if (dlat_pool) memcpy(dlat_pool + pg * nc, gc + pg * nc, sizeof(double) * nc);
    if (dkp_pool) memcpy(dkp_pool + pg * npp, gp + pg * npp, sizeof(double) * npp);
  }
  free(gc); free(gp); free(listed);
  return 0;
}
