// paged_plan.cpp -- host planner of the paged history backward: block tables,
// lengths and packed query rows -> the plan words of paged.hpp.
//
// Follows the host-side preparation that ruDNN 0.1.43
// src/paged_attention/ordered_kernel.rs `history_backward` relies on: the
// listed history pages, the physical page -> (sequence, logical page) links
// (a page reached from several sequences sums over all of them), the
// sequence -> query-row CSR in the original packed row order, and each
// sequence's largest query position (a token past it is seen by no row of the
// sequence under the causal rule).  Its per-token row pruning (monotonic
// flags, block maxima) is replaced by a per-chunk test in the kernel, which
// reads every row's position.
#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "attn_bwd.h"
#include "paged.hpp"

namespace attn {
void set_last_error(const char *msg);
}

namespace {

using namespace attn::plan;
using attn::kQBlockRows;

int perr(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  attn::set_last_error(buf);
  return code;
}

int64_t npages_of(int64_t len, int64_t ps) { return (len + ps - 1) / ps; }

// Checks shared by plan_words and plan_build (the parts that need no table).
int check_dims(int32_t nseq, const int32_t *seq_lens, int32_t max_pages, int32_t nq,
               int32_t heads, int32_t kv_heads, int32_t page_size, int32_t pool_pages) {
  if (nseq < 0 || nq < 0 || max_pages < 0 || pool_pages < 0)
    return perr(ATTN_E_INVALID, "paged plan: negative count");
  if (page_size < 1) return perr(ATTN_E_INVALID, "paged plan: page_size must be >= 1");
  if (heads < 1 || kv_heads < 1 || heads % kv_heads != 0)
    return perr(ATTN_E_INVALID, "paged plan: heads (%d) must be a positive multiple of kv_heads (%d)",
                heads, kv_heads);
  if (nseq > 0 && !seq_lens) return perr(ATTN_E_INVALID, "paged plan: seq_lens is NULL");
  if ((int64_t)pool_pages * page_size > INT32_MAX / 2)
    return perr(ATTN_E_UNSUPPORTED, "paged plan: pool of %lld slots exceeds 2^30",
                (long long)pool_pages * page_size);
  if ((int64_t)nq * heads > INT32_MAX / 4)
    return perr(ATTN_E_UNSUPPORTED, "paged plan: nq * heads exceeds 2^29");
  for (int32_t s = 0; s < nseq; ++s)
    if (seq_lens[s] < 0 || npages_of(seq_lens[s], page_size) > max_pages)
      return perr(ATTN_E_INVALID, "paged plan: sequence %d has length %d, more than %d pages of %d",
                  s, seq_lens[s], max_pages, page_size);
  return ATTN_OK;
}

// Upper bound on the plan size (exact when no page is shared and every page
// fits an item by itself).
int64_t words_bound(int32_t nseq, const int32_t *seq_lens, int32_t nq, int32_t heads,
                    int32_t kv_heads, int32_t page_size, int32_t pool_pages) {
  int64_t refs = 0, tokens = 0, maxlen = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    refs += npages_of(seq_lens[s], page_size);
    tokens += seq_lens[s];
    maxlen = std::max<int64_t>(maxlen, seq_lens[s]);
  }
  const int64_t pieces = npages_of(page_size, kItemSlots);
  const int64_t items = refs * pieces, links = refs * pieces;
  const int64_t qh = (int64_t)nq * (heads / kv_heads);
  using attn::kQBlockRows;
  using attn::kQPieceTokens;
  const int64_t qblk = (qh + kQBlockRows - 1) / kQBlockRows + nseq;
  const int64_t qpieces = qblk * std::max<int64_t>(1, (maxlen + kQPieceTokens - 1) / kQPieceTokens);
  return HEADER_WORDS + (items + 1) + items * kItemSlots + links * (1 + LINK_INFO_WORDS + kItemSlots) +
         (nseq + 1) + 2 * qh + 2 * nseq + std::min<int64_t>(refs, pool_pages) + (nseq + 1) +
         tokens + 2 * qblk + 4 * qpieces + qblk + 1;
}

}  // namespace

extern "C" int64_t attn_bwd_paged_plan_words(int32_t nseq, const int32_t *seq_lens,
                                             int32_t max_pages_per_seq, int32_t nq, int32_t heads,
                                             int32_t kv_heads, int32_t page_size,
                                             int32_t pool_pages) {
  if (check_dims(nseq, seq_lens, max_pages_per_seq, nq, heads, kv_heads, page_size, pool_pages) !=
      ATTN_OK)
    return -1;
  const int64_t w = words_bound(nseq, seq_lens, nq, heads, kv_heads, page_size, pool_pages);
  if (w > INT32_MAX) {
    perr(ATTN_E_UNSUPPORTED, "paged plan: %lld words exceed 2^31", (long long)w);
    return -1;
  }
  return w;
}

extern "C" int attn_bwd_paged_plan_build(int32_t nseq, const int32_t *seq_lens,
                                         const int32_t *block_table, int32_t max_pages_per_seq,
                                         int32_t nq, const int32_t *query_seq,
                                         const int32_t *query_pos, int32_t heads, int32_t kv_heads,
                                         int32_t page_size, int32_t pool_pages, int32_t *plan_out,
                                         int64_t plan_words) {
  const int rc = check_dims(nseq, seq_lens, max_pages_per_seq, nq, heads, kv_heads, page_size,
                            pool_pages);
  if (rc != ATTN_OK) return rc;
  if (!plan_out) return perr(ATTN_E_INVALID, "paged plan: plan_out is NULL");
  if (nq > 0 && (!query_seq || !query_pos))
    return perr(ATTN_E_INVALID, "paged plan: query_seq / query_pos is NULL");
  const int64_t bound = words_bound(nseq, seq_lens, nq, heads, kv_heads, page_size, pool_pages);
  if (plan_words < bound)
    return perr(ATTN_E_INVALID, "paged plan: plan_words %lld < %lld (attn_bwd_paged_plan_words)",
                (long long)plan_words, (long long)bound);
  const int64_t ps = page_size, mp = max_pages_per_seq;

  // Page -> links, in (sequence, logical page) order.
  struct Link { int32_t seq, lpage; };
  std::vector<std::vector<Link>> links_of((size_t)pool_pages);
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t np = npages_of(seq_lens[s], ps);
    if (np > 0 && !block_table) return perr(ATTN_E_INVALID, "paged plan: block_table is NULL");
    for (int64_t lp = 0; lp < np; ++lp) {
      const int32_t pg = block_table[s * mp + lp];
      if (pg < 0 || pg >= pool_pages)
        return perr(ATTN_E_INVALID, "paged plan: block_table[%d][%lld] = %d outside [0, %d)", s,
                    (long long)lp, pg, pool_pages);
      links_of[pg].push_back(Link{s, (int32_t)lp});
    }
  }
  for (int32_t r = 0; r < nq; ++r) {
    if (query_seq[r] < 0 || query_seq[r] >= nseq)
      return perr(ATTN_E_INVALID, "paged plan: query_seq[%d] = %d outside [0, %d)", r, query_seq[r],
                  nseq);
    if (query_pos[r] < 0)
      return perr(ATTN_E_INVALID, "paged plan: query_pos[%d] = %d is negative", r, query_pos[r]);
  }

  // Items: listed pages in first-reference order (sequence-major), grouped
  // while they share the same list of linked sequences.
  struct Piece { int32_t page, off0; };  // slots [off0, off0 + min(ps, 128)) of a page
  std::vector<std::vector<Piece>> items;
  std::vector<const std::vector<Link> *> item_sig;
  std::vector<char> seen((size_t)pool_pages, 0);
  const int per_item = ps <= kItemSlots ? (int)(kItemSlots / ps) : 1;
  auto same_sig = [](const std::vector<Link> &a, const std::vector<Link> &b) {
    if (a.size() != b.size()) return false;
    for (size_t i = 0; i < a.size(); ++i)
      if (a[i].seq != b[i].seq) return false;
    return true;
  };
  std::vector<int32_t> listed;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t np = npages_of(seq_lens[s], ps);
    for (int64_t lp = 0; lp < np; ++lp) {
      const int32_t pg = block_table[s * mp + lp];
      if (seen[pg]) continue;
      seen[pg] = 1;
      listed.push_back(pg);
      const std::vector<Link> &sig = links_of[pg];
      if (ps > kItemSlots) {
        for (int64_t o = 0; o < ps; o += kItemSlots) {
          items.push_back({Piece{pg, (int32_t)o}});
          item_sig.push_back(&sig);
        }
      } else if (!items.empty() && (int)items.back().size() < per_item &&
                 same_sig(*item_sig.back(), sig)) {
        items.back().push_back(Piece{pg, 0});
      } else {
        items.push_back({Piece{pg, 0}});
        item_sig.push_back(&sig);
      }
    }
  }
  std::sort(listed.begin(), listed.end());

  // Sequence -> query-head rows.
  const int32_t group = heads / kv_heads;
  std::vector<int32_t> rows_cnt((size_t)nseq + 1, 0);
  for (int32_t r = 0; r < nq; ++r) ++rows_cnt[query_seq[r] + 1];
  std::vector<int64_t> row_start((size_t)nseq + 1, 0);
  for (int32_t s = 0; s < nseq; ++s) row_start[s + 1] = row_start[s] + rows_cnt[s + 1];
  std::vector<int32_t> seq_rows((size_t)nq);
  {
    std::vector<int64_t> fill(row_start.begin(), row_start.end() - 1);
    for (int32_t r = 0; r < nq; ++r) seq_rows[fill[query_seq[r]]++] = r;  // ascending r
  }

  // Smallest / largest query position of each sequence (INT32_MAX / -1 without rows).
  std::vector<int32_t> seq_minpos((size_t)nseq, INT32_MAX), seq_maxpos((size_t)nseq, -1);
  for (int32_t r = 0; r < nq; ++r) {
    const int32_t s = query_seq[r];
    seq_minpos[s] = std::min(seq_minpos[s], query_pos[r]);
    seq_maxpos[s] = std::max(seq_maxpos[s], query_pos[r]);
  }

  // Emit.
  int32_t *w = plan_out;
  std::fill(w, w + HEADER_WORDS, 0);
  int64_t at = HEADER_WORDS;
  const int64_t n_items = (int64_t)items.size();
  w[W_OFF_ITEM_LINKS] = (int32_t)at;
  at += n_items + 1;
  w[W_OFF_ITEM_SLOTS] = (int32_t)at;
  at += n_items * kItemSlots;
  // Links are counted while emitting; reserve the bound's worth after the slots.
  int64_t max_links = 0;
  for (auto *sig : item_sig) max_links += (int64_t)sig->size();
  w[W_OFF_LINK_SEQ] = (int32_t)at;
  at += max_links;
  w[W_OFF_LINK_INFO] = (int32_t)at;
  at += max_links * LINK_INFO_WORDS;
  w[W_OFF_LINK_TOK] = (int32_t)at;
  at += max_links * kItemSlots;
  w[W_OFF_SEQ_QH] = (int32_t)at;
  at += nseq + 1;
  const int64_t n_qh = (int64_t)nq * group;
  w[W_OFF_QH_RH] = (int32_t)at;
  at += n_qh;
  w[W_OFF_QH_POS] = (int32_t)at;
  at += n_qh;
  w[W_OFF_SEQ_MAXPOS] = (int32_t)at;
  at += nseq;
  w[W_OFF_LISTED] = (int32_t)at;
  at += (int64_t)listed.size();
  w[W_OFF_SEQ_MINPOS] = (int32_t)at;
  at += nseq;
  int64_t tokens = 0;
  for (int32_t s = 0; s < nseq; ++s) tokens += seq_lens[s];
  w[W_OFF_SEQ_TOK] = (int32_t)at;
  at += nseq + 1;
  w[W_OFF_TOK_SLOT] = (int32_t)at;
  at += tokens;
  // Query blocks: 128 qh rows of one sequence each, the sequences whose rows
  // see the most tokens first (the heaviest workgroups start first).
  std::vector<std::pair<int64_t, int32_t>> order;  // (-visible tokens, sequence)
  for (int32_t s = 0; s < nseq; ++s) {
    if (rows_cnt[s + 1] == 0) continue;
    int32_t mx = -1;
    for (int64_t k = row_start[s]; k < row_start[s + 1]; ++k) mx = std::max(mx, query_pos[seq_rows[k]]);
    order.push_back({-std::min<int64_t>(seq_lens[s], (int64_t)mx + 1), s});
  }
  std::stable_sort(order.begin(), order.end(),
                   [](const std::pair<int64_t, int32_t> &a, const std::pair<int64_t, int32_t> &b) {
                     return a.first < b.first;
                   });
  int64_t n_qblk = 0;
  for (auto &o : order) n_qblk += (rows_cnt[o.second + 1] * (int64_t)group + kQBlockRows - 1) / kQBlockRows;
  w[W_OFF_QBLK] = (int32_t)at;
  at += 2 * n_qblk;
  // Query pieces: each block's token range [0, len) in pieces of at most
  // kQPieceTokens (an empty sequence still gets one, empty, piece).
  using attn::kQPieceTokens;
  int64_t n_qpiece = 0;
  for (auto &o : order) {
    const int64_t nb = (rows_cnt[o.second + 1] * (int64_t)group + kQBlockRows - 1) / kQBlockRows;
    n_qpiece += nb * std::max<int64_t>(1, (seq_lens[o.second] + kQPieceTokens - 1) / kQPieceTokens);
  }
  w[W_OFF_QPIECE] = (int32_t)at;
  at += 3 * n_qpiece;
  w[W_OFF_QBLK_PIECE] = (int32_t)at;
  at += n_qblk + 1;
  w[W_OFF_QPIECE_ORDER] = (int32_t)at;
  at += n_qpiece;
  if (at > plan_words) return perr(ATTN_E_INVALID, "paged plan: internal size error");

  int32_t *item_links = w + w[W_OFF_ITEM_LINKS], *item_slots = w + w[W_OFF_ITEM_SLOTS];
  int32_t *link_seq = w + w[W_OFF_LINK_SEQ], *link_info = w + w[W_OFF_LINK_INFO];
  int32_t *link_tok = w + w[W_OFF_LINK_TOK];
  int64_t n_links = 0;
  std::vector<int32_t> lane_page(kItemSlots), lane_off(kItemSlots);
  std::vector<char> live(kItemSlots);
  for (int64_t it = 0; it < n_items; ++it) {
    const std::vector<Piece> &pcs = items[it];
    for (int i = 0; i < kItemSlots; ++i) {
      lane_page[i] = -1;
      if (ps > kItemSlots) {
        const int64_t o = pcs[0].off0 + i;
        if (o < ps) { lane_page[i] = pcs[0].page; lane_off[i] = (int32_t)o; }
      } else if (i / ps < (int64_t)pcs.size()) {
        lane_page[i] = pcs[i / ps].page;
        lane_off[i] = (int32_t)(i % ps);
      }
      live[i] = 0;
    }
    item_links[it] = (int32_t)n_links;
    const std::vector<Link> &sig = *item_sig[it];
    for (size_t j = 0; j < sig.size(); ++j) {
      const int32_t s = sig[j].seq;
      int32_t *tok = link_tok + n_links * kItemSlots;
      int32_t tmin = INT32_MAX, tmax = -1, all = 1;
      for (int i = 0; i < kItemSlots; ++i) {
        int32_t t = -1;
        if (lane_page[i] >= 0) {
          const Link &l = links_of[lane_page[i]][j];  // same sequence list on every page
          const int64_t tt = (int64_t)l.lpage * ps + lane_off[i];
          if (tt < seq_lens[s]) t = (int32_t)tt;
        }
        tok[i] = t;
        if (t >= 0) {
          live[i] = 1;
          tmin = std::min(tmin, t);
          tmax = std::max(tmax, t);
        } else {
          all = 0;
        }
      }
      if (tmax < 0) continue;  // no token of this item inside the sequence
      link_seq[n_links] = s;
      int32_t *info = link_info + n_links * LINK_INFO_WORDS;
      info[LI_MIN_TOK] = tmin;
      info[LI_MAX_TOK] = tmax;
      info[LI_ALL_VALID] = all;
      info[LI_QH0] = (int32_t)(row_start[s] * group);
      info[LI_NQH] = (int32_t)(rows_cnt[s + 1] * (int64_t)group);
      info[LI_MINPOS] = seq_minpos[s];
      info[LI_MAXPOS] = seq_maxpos[s];
      info[LI_SEQ] = s;
      ++n_links;
    }
    for (int i = 0; i < kItemSlots; ++i)
      item_slots[it * kItemSlots + i] =
          lane_page[i] < 0 ? -1 : (int32_t)(((int64_t)lane_page[i] * ps + lane_off[i]) * 2 + live[i]);
  }
  item_links[n_items] = (int32_t)n_links;

  int32_t *seq_qh = w + w[W_OFF_SEQ_QH], *qh_rh = w + w[W_OFF_QH_RH];
  int32_t *qh_pos = w + w[W_OFF_QH_POS], *seq_max = w + w[W_OFF_SEQ_MAXPOS];
  int32_t *seq_min = w + w[W_OFF_SEQ_MINPOS];
  for (int32_t s = 0; s <= nseq; ++s) seq_qh[s] = (int32_t)(row_start[s] * group);
  for (int32_t s = 0; s < nseq; ++s) {
    for (int64_t k = row_start[s]; k < row_start[s + 1]; ++k) {
      const int32_t r = seq_rows[k];
      for (int32_t hh = 0; hh < group; ++hh) {
        qh_rh[k * group + hh] = r * heads + hh;
        qh_pos[k * group + hh] = query_pos[r];
      }
    }
    seq_max[s] = seq_maxpos[s];
    seq_min[s] = seq_minpos[s];
  }
  std::copy(listed.begin(), listed.end(), w + w[W_OFF_LISTED]);
  int32_t *seq_tok = w + w[W_OFF_SEQ_TOK], *tok_slot = w + w[W_OFF_TOK_SLOT];
  {
    int64_t k = 0;
    for (int32_t s = 0; s < nseq; ++s) {
      seq_tok[s] = (int32_t)k;
      for (int64_t t = 0; t < seq_lens[s]; ++t)
        tok_slot[k++] = (int32_t)((int64_t)block_table[s * mp + t / ps] * ps + t % ps);
    }
    seq_tok[nseq] = (int32_t)k;
  }

  {
    int32_t *qb = w + w[W_OFF_QBLK];
    int64_t k = 0;
    for (auto &o : order) {
      const int64_t nqh = rows_cnt[o.second + 1] * (int64_t)group;
      for (int64_t b = 0; b < nqh; b += kQBlockRows) {
        qb[2 * k] = o.second;
        qb[2 * k + 1] = (int32_t)b;
        ++k;
      }
    }
  }
  w[W_QBLK] = (int32_t)n_qblk;
  {
    const int32_t *qb = w + w[W_OFF_QBLK];
    int32_t *qp = w + w[W_OFF_QPIECE], *qbp = w + w[W_OFF_QBLK_PIECE];
    int32_t *qord = w + w[W_OFF_QPIECE_ORDER];
    int64_t k = 0;
    for (int64_t b = 0; b < n_qblk; ++b) {
      qbp[b] = (int32_t)k;
      const int32_t len = seq_lens[qb[2 * b]];
      int32_t t = 0;
      do {
        const int32_t e = (int32_t)std::min<int64_t>(len, (int64_t)t + kQPieceTokens);
        qp[3 * k] = (int32_t)b;
        qp[3 * k + 1] = t;
        qp[3 * k + 2] = e;
        ++k;
        t = e;
      } while (t < len);
    }
    qbp[n_qblk] = (int32_t)k;
    // Split grid order: the longest pieces first (ties in piece order).
    std::vector<int32_t> ids(k);
    for (int64_t i = 0; i < k; ++i) ids[i] = (int32_t)i;
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b2) {
      return qp[3 * a + 2] - qp[3 * a + 1] > qp[3 * b2 + 2] - qp[3 * b2 + 1];
    });
    std::copy(ids.begin(), ids.end(), qord);
    w[W_QPIECES] = (int32_t)k;
  }
  w[W_MAGIC] = kMagic;
  w[W_WORDS] = (int32_t)at;
  w[W_NSEQ] = nseq;
  w[W_NQ] = nq;
  w[W_HEADS] = heads;
  w[W_KV_HEADS] = kv_heads;
  w[W_PAGE_SIZE] = page_size;
  w[W_POOL_PAGES] = pool_pages;
  w[W_ITEMS] = (int32_t)n_items;
  w[W_LINKS] = (int32_t)n_links;
  w[W_QH] = (int32_t)n_qh;
  w[W_LISTED] = (int32_t)listed.size();
  w[W_TOKENS] = (int32_t)tokens;
  return ATTN_OK;
}
