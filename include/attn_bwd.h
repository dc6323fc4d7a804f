/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) scaled dot-product attention
 * backward library (libattn_bwd.so).
 *
 * The operation (dense):
 *   S  = scale * Q K^T (+ bias), masked;  P = row softmax(S);
 *   dV = P^T dY;  dP = dY V^T;  dS = P * (dP - rowsum(P * dP)) * scale;
 *   dQ = dS K;    dK = dS^T Q.
 * as defined by docs.rs rlx-cpu 0.2.17, src/attention_bwd.rs
 * (`backward_dense_head_all`, `attention_backward_all`, `apply_synthetic_mask`),
 * with the strided layout and the numeric mask / wrt codes of docs.rs rlx-wgpu
 * 0.2.1, src/kernels/attention_bwd.wgsl (`Params`, `mask_score`).
 *
 * The operation (paged): dK / dV of a grouped-query attention whose keys and
 * values live in a page-permuted pool, given the per-row statistics
 * (max, denominator, rowsum(P * dP)), as defined by docs.rs ruDNN 0.1.43,
 * src/paged_attention/ordered_kernel.rs (`history_backward`).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are GPU memory the caller allocated; "host"
 *     pointers are CPU memory.  The library never allocates, frees or keeps
 *     any of them, and holds no state between calls.
 *   - `stream` is a hipStream_t passed as void*.  Work is enqueued on it and the
 *     call returns without synchronising: inputs must stay alive, and outputs
 *     must not be read, until the stream has passed this point.
 *   - Return value: ATTN_OK (0) or a negative status.  On a negative status
 *     nothing was enqueued and attn_bwd_last_error() describes the problem.
 *   - Outputs are fully determined by the inputs: no atomics, fixed reduction
 *     orders, bit-identical from run to run.
 *   - Calls on different streams may overlap; calls that share an output or a
 *     workspace must be ordered by the caller.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, dY and of every gradient output. */
enum { ATTN_F32 = 0, ATTN_BF16 = 1 };

/* Which gradients to produce.  0..2 are the `wrt` codes of rlx-wgpu
 * attention_bwd.wgsl (0 = dQ, 1 = dK, 2 = dV); 3 asks for all three from one
 * score recompute, as rlx-cpu `attention_backward_all`. */
enum { ATTN_WRT_Q = 0, ATTN_WRT_K = 1, ATTN_WRT_V = 2, ATTN_WRT_ALL = 3 };

/* Mask kinds: the MaskKind codes of rlx-wgpu `mask_score`.
 *   NONE   every key visible.
 *   CAUSAL query i (absolute position a = max(Sk - Sq, 0) + i) sees keys j <= a
 *          (rlx-cpu `apply_synthetic_mask`).
 *   KEYPAD key j hidden when mask[b,h,i,j] < mask_threshold ("Custom").
 *   WINDOW sees keys max(a - window, 0) <= j <= a ("SlidingWindow(w)").
 *   BIAS   mask[b,h,i,j] is added to the scaled score ("Bias").
 * Hidden keys are excluded from the softmax; a row with no visible key has
 * P = 0, contributes nothing, and its dQ row is 0. */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_KEYPAD = 2,
  ATTN_MASK_WINDOW = 3,
  ATTN_MASK_BIAS = 4
};
/* mask_flags bit: also apply the causal rule, after KEYPAD or BIAS. */
#define ATTN_MASK_FLAG_CAUSAL 0x1

enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* bad enum, size, pointer, stride, aliasing or plan */
  ATTN_E_UNSUPPORTED = -2, /* head_dim not in {32, 64, 128}, d not contiguous, rows not 16-byte aligned */
  ATTN_E_WORKSPACE = -3,   /* workspace missing or smaller than attn_bwd_workspace_bytes() */
  ATTN_E_HIP = -4          /* the HIP runtime refused a launch */
};

/* Dense arguments.  Tensors are [B, S, H, D] in element strides (b, s, h) with
 * d contiguous (stride 1); [B, H, S, D] is the same with other strides
 * (rlx-wgpu `Params` carries per-tensor batch / head / seq strides). */
typedef struct attn_bwd_args {
  int32_t dtype;           /* ATTN_F32 or ATTN_BF16, for all seven tensors */
  int32_t wrt;             /* ATTN_WRT_* */
  int64_t B, H, Sq, Sk, D; /* D in {32, 64, 128}; Sq, Sk < 2^30 */
  const void *q, *k, *v, *dy; /* device, read only. q, dy: [B,Sq,H,D]; k, v: [B,Sk,H,D] */
  void *dq, *dk, *dv;         /* device outputs; required iff `wrt` asks for them, else ignored */
  int64_t q_stride[3], k_stride[3], v_stride[3], dy_stride[3]; /* (b, s, h) element strides, >= 0 */
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int32_t mask_kind;       /* ATTN_MASK_* */
  int32_t mask_flags;      /* 0 or ATTN_MASK_FLAG_CAUSAL (KEYPAD / BIAS only) */
  int64_t window;          /* WINDOW only, >= 0: keeps window + 1 keys */
  const float *mask;       /* device fp32, KEYPAD validity or BIAS values; else ignored */
  int64_t mask_stride[4];  /* (b, h, i, j) element strides, 0 = broadcast ([B,Sk] padding: {Sk,0,0,1}) */
  float mask_threshold;    /* KEYPAD: key hidden iff value < threshold */
  float scale;             /* 2^-64 <= |scale| <= 2^64 (else ATTN_E_UNSUPPORTED; NaN or inf:
                              ATTN_E_INVALID); callers usually pass (float)(1/sqrt(D)) */
  void *workspace;         /* device, >= attn_bwd_workspace_bytes(B, H, Sq) bytes, 256-byte aligned */
  size_t workspace_bytes;
  int64_t Hkv;             /* K / V heads (grouped-query attention); 0 means H.  H must be a
                              multiple of Hkv; query head h reads K / V head h / (H / Hkv);
                              k, v, dk, dv are [B, Sk, Hkv, D] and dk, dv sum over each group */
} attn_bwd_args;

/* Bytes of device workspace attn_bwd needs: four fp32 planes of B*H*Sq row
 * statistics, each padded to 256 bytes.  Plane 0 = row max m of the scaled
 * scores, plane 1 = denominator l = sum exp(s - m), plane 2 = delta =
 * rowsum(P * dP), plane 3 = internal (-lse / scale, lse = m + ln l).  Row (b, h, i)
 * sits at index (b * H + h) * Sq + i.  An empty row holds m = -inf, l = 0,
 * delta = 0.  Returns 0 for negative sizes, and SIZE_MAX when the planes would
 * exceed 2^60 bytes (sizes attn_bwd rejects). */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq);

/* A larger workspace that also holds the split form of the passes (all but
 * the dQ pass that forms a forward's statistics): the four planes above, then
 * partial results of up to 16 pieces per row (max(D, 4) fp32 per query row for
 * the row-statistics and dQ passes, 2 D + 8 for the fused bf16 statistics + dQ
 * pass, 2 D per key row for dK / dV).  With
 * workspace_bytes >= this size the library cuts a pass's streamed axis (keys
 * for the query-major passes, queries for dK / dV) into pieces of whole chunks
 * (at least four each) when its workgroups would leave most compute units
 * idle (few queries against many keys, or the reverse), and merges the
 * pieces' results in piece order: the same sums in another order, so the
 * outputs equal the one-workgroup-per-block form's up to rounding, and reruns
 * with the same workspace size on the same device are bit-identical.  Returns
 * attn_bwd_workspace_bytes() where no split is possible (fewer than 256 keys
 * and queries), 0 for negative sizes or D outside (0, 4096]. */
size_t attn_bwd_split_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D);

/* The whole dense backward, as `wrt` asks.  bf16: one query-major pass
 * computes the row statistics and dQ together (attn_bwd_stats_dq), then the
 * KV-major pass writes dK / dV.  fp32: row statistics, dK / dV, dQ (the three
 * stages below).  Every element of every requested output is written (no pre-zeroing
 * needed, as rlx-cpu `attention_backward_all`); no output may overlap any
 * input, another output or the workspace.  B, H, Sq or Sk = 0 is valid: the
 * requested outputs that have elements are then written with zeros. */
int attn_bwd(const attn_bwd_args *a, void *stream);

/* attn_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results, but `workspace` / `workspace_bytes` are ignored and
 * the row statistics live in a static device array the library holds on each
 * GPU (16 MiB, from the first use of the library's code on that GPU until the
 * process ends); it runs the form attn_bwd takes with a workspace of exactly
 * attn_bwd_workspace_bytes() (never the split form), so the two give the same
 * bits.  B * H * Sq must be at most 2^20 rows, else ATTN_E_WORKSPACE
 * (before any HIP call).  The array's device address is looked up once per
 * device, on the device current on the calling thread, which must be the
 * stream's device.  The call allocates and frees nothing.  All calls on one
 * GPU share the array: calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller. */
int attn_bwd_noalloc(const attn_bwd_args *a, void *stream);

/* The three stages of attn_bwd, for callers that time or schedule them one by
 * one.  They take the same arguments and validation.  Run them in this order
 * on one stream: row_stats fills the workspace statistics; kv writes dK / dV
 * (those `wrt` asks for) from them; dq writes dQ (if asked) from them. */
int attn_bwd_row_stats(const attn_bwd_args *a, void *stream);
int attn_bwd_kv(const attn_bwd_args *a, void *stream);
int attn_bwd_dq(const attn_bwd_args *a, void *stream);

/* Row statistics and dQ in one query-major pass (rlx-cpu
 * `backward_dense_head_all`: dS = P (dP - rowsum(P dP)) scale, dQ = dS K,
 * with rowsum(P dP) found in the same pass: dQ_i = scale (A_i - delta_i B_i)
 * / l_i, A_i = sum_j p~_ij dP_ij K_j, B_i = sum_j p~_ij K_j).  Same arguments
 * and validation as attn_bwd.  It fills the workspace statistics (as
 * attn_bwd_row_stats does, up to rounding: it takes keys 64 at a time, the
 * row-statistics pass 32) and writes dQ if `wrt` asks for it; attn_bwd_kv may
 * follow on the same stream, which is what attn_bwd does for bf16 (same bits).
 * bf16 runs one kernel; fp32 runs attn_bwd_row_stats then attn_bwd_dq. */
int attn_bwd_stats_dq(const attn_bwd_args *a, void *stream);

/* ------------------------------------------------------------------------
 * Paged, grouped-query history backward (dK / dV only), ruDNN 0.1.43
 * src/paged_attention/ordered_kernel.rs `history_backward`.
 *
 * Sequence s has seq_lens[s] tokens; its token t lives in pool slot
 * block_table[s * max_pages_per_seq + t / page_size] * page_size + t % page_size.
 * Query row r (0 <= r < nq, rows packed in any order) belongs to sequence
 * query_seq[r] at position query_pos[r]; with `causal` it sees the tokens
 * t <= query_pos[r] of its sequence, otherwise all of them.  Query head h
 * reads KV head h / (heads / kv_heads).  For every (slot, KV head g) of every
 * listed page (a page some sequence reaches below its length):
 *   dK[slot, g] = sum over links (s, logical page) of the page, rows r of s
 *                 that see the slot's token, heads h of group g, with
 *                 denominator l > 0:  ds * q[r, h]
 *   dV[slot, g] = ... same sum of p * dY[r, h]
 *   p  = exp(scale * q[r,h] . k[slot,g] - m) / l,
 *   ds = p * (dY[r,h] . v[slot,g] - delta) * scale,
 * with (m, l, delta) = stats[r, h, 0..2] (supplied, as on the pages).  Tail
 * slots of listed pages get +0; slots of unlisted pages are left untouched.
 * K / V rows of slots no link reaches are never read (they may hold NaN).
 * Each output element is written once, by one workgroup, in a fixed order.
 *
 * Host planning is split from the launch (the pages prepare their page and
 * row tables on the host too): attn_bwd_paged_plan_words() bounds the plan
 * size, attn_bwd_paged_plan_build() fills host int32 words, the caller copies
 * them to device memory and passes both copies to attn_bwd_paged().  A plan
 * may be reused for any call with the same tables and geometry. */

/* Upper bound on the int32 words of a plan, or -1 (see attn_bwd_last_error)
 * for inconsistent sizes.  seq_lens: host [nseq]. */
int64_t attn_bwd_paged_plan_words(int32_t nseq, const int32_t *seq_lens, int32_t max_pages_per_seq,
                                  int32_t nq, int32_t heads, int32_t kv_heads, int32_t page_size,
                                  int32_t pool_pages);

/* Builds the plan into plan_out (host, plan_words words).  All arrays are host
 * memory: seq_lens [nseq], block_table [nseq, max_pages_per_seq] (only the
 * first ceil(len / page_size) entries of a row are read; each in
 * [0, pool_pages)), query_seq / query_pos [nq] (query_seq in [0, nseq),
 * query_pos >= 0).  Word 1 of the result is the number of words used.
 * ATTN_E_INVALID on any inconsistency; nothing is enqueued anywhere. */
int attn_bwd_paged_plan_build(int32_t nseq, const int32_t *seq_lens, const int32_t *block_table,
                              int32_t max_pages_per_seq, int32_t nq, const int32_t *query_seq,
                              const int32_t *query_pos, int32_t heads, int32_t kv_heads,
                              int32_t page_size, int32_t pool_pages, int32_t *plan_out,
                              int64_t plan_words);

typedef struct attn_bwd_paged_args {
  int32_t dtype;      /* ATTN_F32 or ATTN_BF16: q, dy, pools and gradient pools */
  int32_t need;       /* bit 0: dK, bit 1: dV (at least one); latent variant: see below */
  int32_t heads, kv_heads, head_dim, page_size, causal; /* head_dim in {32, 64, 128} (latent
                                                           variant: see below); causal 0 / 1 */
  int32_t nq, pool_pages;                /* must match the plan */
  float scale;                           /* 2^-64 <= |scale| <= 2^64 */
  const void *q, *dy;                    /* device [nq, heads, head_dim], contiguous */
  const void *k_pool, *v_pool;           /* device [pool_pages * page_size, kv_heads, head_dim] */
  const float *stats;                    /* device [nq, heads, 3] = (max, denominator, delta) */
  const int32_t *plan_host;              /* host plan words (read during the call) */
  const int32_t *plan;                   /* device copy of the same words (read by the kernel) */
  void *dk_pool, *dv_pool;               /* device, same shape as the pools; written only at
                                            slots of listed pages; NULL allowed iff not in `need` */
  /* Latent (MLA) variant, ruDNN history_backward with its `mla` switch: set
   * mla = 1.  Then k_pool holds each slot's latent row c (width head_dim, which
   * is both key and value; v_pool and dv_pool are not used), kp_pool the
   * position keys [pool_pages * page_size, kv_heads, position_dim], qp the
   * queries' position parts [nq, heads, position_dim]; q and dy keep width
   * head_dim.  Per visible (row, head, token):
   *   s  = scale * (q . c + qp . kp),  p = exp(s - m) / l,
   *   ds = p * (dY . c - delta) * scale,
   *   dk_pool[slot, g]  (the latent's gradient) += ds * q + p * dY,
   *   dkp_pool[slot, g] += ds * qp.
   * need: bit 0 the latent's gradient, bit 2 the position keys' (bit 1 is
   * invalid).  head_dim in {64, 128} (bf16 also 192 or 256, streamed in 32-row
   * chunks), position_dim in {0, 32, 64}.  The query
   * side (row statistics, dQ) does not take the latent variant.  mla = 0: the
   * fields below are ignored. */
  int32_t mla, position_dim;
  const void *qp, *kp_pool;              /* device, 16-byte aligned, contiguous */
  void *dkp_pool;                        /* device [pool_pages * page_size, kv_heads, position_dim] */
  /* Query side only (attn_bwd_paged_row_stats / attn_bwd_paged_dq): NULL, or a
   * device workspace of q_workspace_bytes >= attn_bwd_paged_q_workspace_bytes()
   * (16-byte aligned, overlapping nothing else).  With it the call runs in split
   * form: each query block's tokens are cut into pieces of at most 1024, one
   * workgroup per piece, and a merge pass combines the pieces in token order,
   * so a long sequence no longer sets the time.  Results equal the direct form
   * up to rounding order; both are bit-identical from run to run. */
  void *q_workspace;
  size_t q_workspace_bytes;
  /* Form of the dK / dV pass of attn_bwd_paged (bf16, not latent; ignored
   * otherwise).  0: chosen by the library, the persistent form (one workgroup
   * per compute unit, each walking a fixed list of (item, KV head) units)
   * when the units outnumber the compute units, else one workgroup per unit;
   * n > 0: the persistent form with n workgroups (rounded down to a multiple
   * of 8, at least 8, at most the units rounded up to 8); -1: one workgroup
   * per unit.  Every form gives identical bits.  Below -1: ATTN_E_INVALID. */
  int32_t kv_workgroups;
  /* Form of attn_bwd_paged_stats_dq (bf16; ignored by the other calls and for
   * fp32).  0: chosen by the library: without q_workspace the direct form (one
   * workgroup per (query block, KV head)); with it, the split form only where
   * the plan's estimated time is lower (a few long sequences: the direct form
   * waits for the longest block; many blocks: the split form pays a fixed
   * cost per piece and the merge).  1: the split form (q_workspace required,
   * else ATTN_E_WORKSPACE); 2: the direct form (q_workspace not used).  The
   * forms differ in rounding order; each is bit-identical from run to run.
   * Other values: ATTN_E_INVALID. */
  int32_t q_form;
} attn_bwd_paged_args;

/* Enqueues the paged backward.  Every device pointer must be 16-byte aligned;
 * the gradient pools may not overlap any input or each other.  The device plan
 * must be an unmodified copy of plan_host.  Trust boundary: the library checks
 * the host copy (magic, header offsets inside the plan, geometry equal to the
 * arguments) but never reads the device copy on the host; the kernels trust
 * its tables, which address the pools.  Every plan attn_bwd_paged_plan_build
 * writes keeps each table inside the plan, each slot inside the pool and each
 * query row inside [0, nq * heads).  A plan with no item does nothing. */
int attn_bwd_paged(const attn_bwd_paged_args *a, void *stream);

/* The query side of the paged backward, for callers without forward
 * statistics (in ruDNN history_backward a separate query-side kernel produces
 * them, one triple per row): the same
 * arguments and plan as attn_bwd_paged, `need` ignored.
 *
 * attn_bwd_paged_row_stats writes `stats` (device [nq, heads, 3] fp32, the
 * argument struct's `stats` is ignored) = (max of the scaled visible scores,
 * denominator sum exp(s - max), delta = sum_t P dP) per (row, head), with
 * P = exp(s - max) / denominator and dP = dY . v; a row that sees no token
 * gets (-inf, 0, 0).  Feed the result to attn_bwd_paged and attn_bwd_paged_dq.
 *
 * attn_bwd_paged_dq writes `dq` (device [nq, heads, head_dim], the element
 * type of q) = sum over the row's visible tokens of dS k, with
 * dS = P (dP - delta) scale from the argument struct's `stats`; a row with a
 * zero denominator gets a zero dQ row.  Every row of `dq` is written.
 *
 * Both reject outputs that overlap an input; the plan, pointers and
 * alignment follow attn_bwd_paged. */
int attn_bwd_paged_row_stats(const attn_bwd_paged_args *a, float *stats, void *stream);

/* Bytes of q_workspace the split form of the query side needs for a plan
 * (host words) and head_dim, for any of the three query-side calls:
 * pieces * kv_heads * 128 rows * (2 head_dim + 8) fp32 (the fused call's
 * partial statistics and two partial accumulators per row; the others use 4
 * or head_dim of those floats).  0 for a buffer that is not a plan. */
size_t attn_bwd_paged_q_workspace_bytes(const int32_t *plan_host, int32_t head_dim);
int attn_bwd_paged_dq(const attn_bwd_paged_args *a, void *dq, void *stream);

/* Both of the above in one call: `stats` as attn_bwd_paged_row_stats writes
 * it and `dq` as attn_bwd_paged_dq would write it from those statistics
 * (rlx-cpu `backward_dense_head_all` forms dS = P (dP - rowsum(P dP)) scale
 * and dQ = dS K; ruDNN `history_backward` takes the statistics from a
 * query-side kernel).  bf16: one pass over the tokens, accumulating
 * A = sum P~ (dP - d) k and B = sum P~ k against the running statistics
 * (P~ = exp(s - running max), d = the running estimate of delta), so that
 * dq = scale (A + (d - delta) B) / denominator; the statistics equal
 * attn_bwd_paged_row_stats's up to rounding, dq equals attn_bwd_paged_dq's
 * from them up to rounding.  fp32: the two calls in sequence.  Outputs must
 * not overlap each other or an input; with q_workspace (split form) the
 * workspace needs attn_bwd_paged_q_workspace_bytes().  Reruns are
 * bit-identical.  Errors as attn_bwd_paged; nothing is launched on error. */
int attn_bwd_paged_stats_dq(const attn_bwd_paged_args *a, float *stats, void *dq, void *stream);

/* The dense backward from what a forward pass saved, instead of recomputing
 * the row statistics: `lse` (device fp32 [B, H, Sq], contiguous) holds, per
 * row, the natural log-sum-exp of its scaled, masked scores (-inf for a row
 * that sees no key), and `out` (device, the element type of q, [B, Sq, H, D]
 * with element strides out_stride[0..2] for (b, s, h)) the forward output O.
 * Then delta = rowsum(dY * O) (= rowsum(P * dP)) and P = exp(s - lse): the
 * dQ kernel forms delta and the row offsets in its prologue (and stops there
 * when dQ is not asked for), then the dK / dV kernel runs, so every `wrt`
 * gives the same bits.  Workspace planes 2 (delta) and 3 are written, planes
 * 0 and 1 are not.  Same arguments and rules as attn_bwd
 * otherwise; lse and out must not overlap the workspace. */
int attn_bwd_from_forward(const attn_bwd_args *a, const float *lse, const void *out,
                          const int64_t *out_stride, void *stream);

/* Thread-local description of the last non-OK status returned on this thread. */
const char *attn_bwd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
