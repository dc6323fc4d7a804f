// paged.hpp -- the plan-word format of the paged history backward and the
// kernel's parameter block, shared by the host planner (paged_plan.cpp), the
// C ABI (abi.cpp) and the kernel (paged_kernels.hip).
//
// The method is ruDNN 0.1.43 src/paged_attention/ordered_kernel.rs
// `history_backward`: every physical KV slot that a sequence lists receives
// dK / dV summed over all (sequence, logical page) links of its page, all
// query rows of each linked sequence that can see the slot's token and all
// query heads of the slot's KV-head group, with one final store per element.
// The pages derive, on the host, a list of history pages, a page -> link CSR
// and a sequence -> row CSR.  The plan here carries the same information
// regrouped for 128-slot MFMA tiles:
//
//   item     up to 128 slots of listed pages that share the same list of
//            linked sequences (in practice: consecutive pages of one
//            sequence, or the pages of a shared prefix); one workgroup per
//            (item, KV head).  Slot entry = physical slot * 2 + live, -1 for
//            an unused lane; live = some link's token at this slot lies
//            inside its sequence (tail slots of a last page are not live:
//            they store zero and their K / V rows are never read).
//   link     one sequence linked to every page of an item: per lane the
//            token position of the slot in that sequence (-1: past its
//            length, or no slot), plus an 8-word record: min / max token,
//            whether all 128 lanes hold a token, and the linked sequence's
//            own facts (its qh rows, smallest and largest row position, the
//            sequence), so that a workgroup learns everything about a link
//            from one record.
//   qh row   the query rows of each sequence in their original packed order,
//            each expanded to its group of query heads (head index minor):
//            rh = row * heads + head-in-group, and the row's position.
//   token    each sequence's tokens in order, as pool slots (the query-side
//            kernels stream a sequence's keys through this table).
//   qblock   a sequence's qh rows cut into blocks of 128, one query-side
//            workgroup per (block, KV head).
//   qpiece   a query block's token range cut into pieces of at most
//            kQPieceTokens tokens, for the query side's split form: one
//            workgroup per (piece, KV head) writes partial results that a
//            merge pass combines in piece order.
#pragma once

#include <stdint.h>

namespace attn {
namespace plan {

constexpr int32_t kMagic = 0x32504241;  // "ABP2"
constexpr int kItemSlots = 128;

enum Word {
  W_MAGIC = 0,
  W_WORDS,       // words actually used by this plan
  W_NSEQ,
  W_NQ,
  W_HEADS,
  W_KV_HEADS,
  W_PAGE_SIZE,
  W_POOL_PAGES,
  W_ITEMS,
  W_LINKS,
  W_QH,          // total query-head rows = nq * heads / kv_heads
  W_LISTED,      // listed physical pages
  W_OFF_ITEM_LINKS,  // [items + 1] CSR into links
  W_OFF_ITEM_SLOTS,  // [items * 128] slot entries
  W_OFF_LINK_SEQ,    // [links] sequence
  W_OFF_LINK_INFO,   // [links * LINK_INFO_WORDS] link records (LI_* below)
  W_OFF_LINK_TOK,    // [links * 128] token per lane, -1 = none
  W_OFF_SEQ_QH,      // [nseq + 1] CSR into qh rows
  W_OFF_QH_RH,       // [qh] row * heads + head-in-group
  W_OFF_QH_POS,      // [qh] position of the row
  W_OFF_SEQ_MAXPOS,  // [nseq] largest position of the sequence's rows, -1 if none
  W_OFF_LISTED,      // [listed] listed physical pages, ascending
  W_OFF_SEQ_MINPOS,  // [nseq] smallest position of the sequence's rows, INT32_MAX if none
  W_OFF_SEQ_TOK,     // [nseq + 1] CSR into the token -> slot table
  W_OFF_TOK_SLOT,    // [sum of lengths] pool slot of each token of each sequence
  W_TOKENS,          // sum of lengths
  W_OFF_QBLK,        // [qblocks * 2] (sequence, first qh row) of each 128-qh-row block,
                     // sequences with more visible tokens first
  W_QBLK,            // number of query blocks
  W_OFF_QPIECE,      // [qpieces * 3] (query block, first token, end token), block-major,
                     // token order within a block
  W_OFF_QBLK_PIECE,  // [qblocks + 1] CSR: the pieces of query block b
  W_OFF_QPIECE_ORDER,  // [qpieces] piece ids, longest first (the split grid's order)
  W_QPIECES,         // number of pieces
  HEADER_WORDS = 32
};

// Link record: the item's smallest / largest token in the sequence, 1 if all
// 128 lanes hold a token; the sequence's first qh row and qh row count, its
// rows' smallest and largest position (INT32_MAX / -1 without rows), the
// sequence.
enum {
  LI_MIN_TOK = 0,
  LI_MAX_TOK,
  LI_ALL_VALID,
  LI_QH0,
  LI_NQH,
  LI_MINPOS,
  LI_MAXPOS,
  LI_SEQ,
  LINK_INFO_WORDS = 8
};

}  // namespace plan

constexpr int kQBlockRows = 128;
constexpr int kQPieceTokens = 1024;  // a multiple of the 32-token chunk

struct PagedParams {
  const void *q, *dy, *k_pool, *v_pool;
  void *dk_pool, *dv_pool;
  // latent variant: q's position part [nq, heads, P], the position keys
  // [slots, kv_heads, P] and their gradient; k_pool is the latent, dk_pool its
  // gradient, v_pool / dv_pool unused
  const void *qp, *kp_pool;
  void *dkp_pool;
  int mla, P, need_dkp;
  float *stats_out;  // query side: statistics written here
  void *dq;          // query side: dQ [nq, heads, D]
  const float *stats;   // [nq, heads, 3] = (max, denominator, delta)
  const int32_t *plan;  // device copy of the plan words
  int heads, kv_heads, group;
  int causal, need_dk, need_dv;
  float scale, scale_log2, inv_scale_log2;
  int items;
  int off_item_links, off_item_slots, off_link_seq, off_link_info, off_link_tok;
  int off_seq_qh, off_qh_rh, off_qh_pos, off_seq_maxpos, off_seq_minpos;
  int off_seq_tok, off_tok_slot, off_qblk, qblocks;
  // query side, split form: pieces and the partial results' workspace
  // (per (piece, KV head, row of the block): 4 floats of statistics or D of dQ)
  int off_qpiece, off_qblk_piece, off_qpiece_order, qpieces;
  float *qws;
};

}  // namespace attn
