// abi.cpp -- the C ABI of libattn_bwd.so (declared in include/attn_bwd.h):
// argument validation, workspace sizing and kernel dispatch for the dense path,
// and validation + dispatch of the paged path (its planner is paged_plan.cpp).
//
// Every check happens on the host before anything is enqueued, so a rejected
// call leaves the stream untouched.  The pages' own interfaces have no error
// path (rlx-cpu panics on a bad slice, rlx-metal `use_gpu` falls back to the
// CPU, rlx-wgpu `attention_bwd` silently returns for head_dim > 128); here
// every unsupported or inconsistent request is an explicit status.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn_bwd.h"
#include "launch.hpp"
#include "paged.hpp"

// The dK / dV kernels start the score accumulators at -lse2 / (scale log2 e),
// so the scale must have an invertible, normal-range magnitude, and scale log2 e
// must stay finite: 2^-64 <= |scale| <= 2^64.
constexpr float kMinScale = 5.421010862427522e-20f;  // 2^-64
constexpr float kMaxScale = 1.8446744073709552e19f;  // 2^64

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Largest byte extent a tensor may have: keeps every offset sum below 2^63.
constexpr int64_t kMaxBytes = (int64_t)1 << 60;

// Bytes of B * H * Sq fp32 values (sizes >= 0), or -1 beyond kMaxBytes.
int64_t stat_bytes(int64_t B, int64_t H, int64_t Sq) {
  int64_t n;
  if (__builtin_mul_overflow(B, H, &n) || __builtin_mul_overflow(n, Sq, &n) ||
      __builtin_mul_overflow(n, (int64_t)sizeof(float), &n) || n > kMaxBytes)
    return -1;
  return n;
}

// One statistics plane, 256-byte aligned; 0 beyond kMaxBytes (validate()
// rejects such sizes before it asks).
size_t plane_bytes(int64_t B, int64_t H, int64_t Sq) {
  const int64_t n = stat_bytes(B, H, Sq);
  return n < 0 ? 0 : align256((size_t)n);
}

// Byte range [lo, hi) covered by a [n0, n1, n2, n3] tensor with element strides
// st[0..3] (last one for the innermost axis, all >= 0); empty if any extent is
// 0.  `ok` turns false when the range exceeds kMaxBytes or the address space
// (the arithmetic is exact: 128-bit).
struct Range {
  uintptr_t lo = 0, hi = 0;
  bool empty() const { return hi <= lo; }
};

Range extent(const void *p, const int64_t n[4], const int64_t st[4], size_t esize, bool &ok) {
  Range r;
  ok = true;
  if (!p) return r;
  __int128 last = 0;
  for (int i = 0; i < 4; ++i) {
    if (n[i] <= 0) return r;
    last += (__int128)(n[i] - 1) * st[i];
  }
  const __int128 bytes = (last + 1) * (__int128)esize;
  if (bytes > kMaxBytes || (__int128)(uintptr_t)p + bytes > (__int128)UINTPTR_MAX) {
    ok = false;
    return r;
  }
  r.lo = (uintptr_t)p;
  r.hi = r.lo + (uintptr_t)bytes;
  return r;
}

bool overlap(const Range &a, const Range &b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

struct Checked {
  attn::DenseParams p;
  bool bf16;
  int D;
  int mode;
  bool want_q, want_k, want_v;
  int nblk_q, nblk_k;
  float *ws_split;  // the split form's region of the workspace, or nullptr
};
}  // namespace

namespace attn {
int device_cus();
}

namespace {
// Split form of the row-statistics, dQ and dK / dV passes.  When a pass's
// workgroups (one per query block and head, or per key block and K / V head)
// would leave most compute units idle (few long rows: few queries against
// many keys, or the reverse), each block's streamed axis is cut into pieces
// of whole chunks (32 keys; 32 or 64 query rows for dK / dV), at least
// kSplitMinChunks each and at most kSplitMaxPieces of them, and a merge
// combines the pieces' partial results in piece order.
constexpr int64_t kSplitMinChunks = 4, kSplitMaxPieces = 16;

// Largest piece count over n rows streamed in chunks of `unit`.
int64_t split_max_pieces(int64_t n, int64_t unit = 32) {
  const int64_t chunks = n / unit + (n % unit != 0);  // no overflow for any n >= 0
  return std::min<int64_t>(kSplitMaxPieces, chunks / kSplitMinChunks);
}

// Pieces for a pass with `blocks` workgroups, or 0 for the
// one-workgroup-per-block form: only when at most half of the compute units
// would be busy.
int split_pieces(int64_t blocks, int64_t max_pieces, int cus) {
  if (max_pieces < 2 || cus <= 0 || blocks <= 0 || 2 * blocks > cus) return 0;
  return (int)std::min<int64_t>(max_pieces, std::max<int64_t>(2, cus / blocks));
}

int validate(const attn_bwd_args *a, Checked &c) {
  if (!a) return fail(ATTN_E_INVALID, "args is NULL");
  if (a->dtype != ATTN_F32 && a->dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32 or ATTN_BF16", a->dtype);
  if (a->wrt < ATTN_WRT_Q || a->wrt > ATTN_WRT_ALL)
    return fail(ATTN_E_INVALID, "wrt %d is not one of ATTN_WRT_*", a->wrt);
  if (a->mask_kind < ATTN_MASK_NONE || a->mask_kind > ATTN_MASK_BIAS)
    return fail(ATTN_E_INVALID, "mask_kind %d is not one of ATTN_MASK_*", a->mask_kind);
  if (a->mask_flags & ~ATTN_MASK_FLAG_CAUSAL)
    return fail(ATTN_E_INVALID, "unknown mask_flags bits 0x%x", a->mask_flags);
  if (a->mask_flags && a->mask_kind != ATTN_MASK_KEYPAD && a->mask_kind != ATTN_MASK_BIAS)
    return fail(ATTN_E_INVALID, "mask_flags only combine with ATTN_MASK_KEYPAD or ATTN_MASK_BIAS");
  if (a->B < 0 || a->H < 0 || a->Sq < 0 || a->Sk < 0)
    return fail(ATTN_E_INVALID, "negative size (B=%lld H=%lld Sq=%lld Sk=%lld)", (long long)a->B,
                (long long)a->H, (long long)a->Sq, (long long)a->Sk);
  if (a->Sq >= (1 << 30) || a->Sk >= (1 << 30))
    return fail(ATTN_E_INVALID, "sequence length must be below 2^30");
  if (a->D != 32 && a->D != 64 && a->D != 128)
    return fail(ATTN_E_UNSUPPORTED, "head_dim %lld is not 32, 64 or 128", (long long)a->D);
  if (!std::isfinite(a->scale)) return fail(ATTN_E_INVALID, "scale is not finite");
  if (std::fabs(a->scale) < kMinScale || std::fabs(a->scale) > kMaxScale)
    return fail(ATTN_E_UNSUPPORTED, "|scale| outside [2^-64, 2^64] (including 0) is not supported");
  if (a->mask_kind == ATTN_MASK_WINDOW && a->window < 0)
    return fail(ATTN_E_INVALID, "window %lld is negative", (long long)a->window);
  if (a->mask_kind == ATTN_MASK_KEYPAD && std::isnan(a->mask_threshold))
    return fail(ATTN_E_INVALID, "mask_threshold is NaN");

  // Query-major kernels: 128 queries per workgroup; the KV-major kernel: 128 keys.
  const int64_t qrows = 128;
  const int64_t nblk_q = (a->Sq + qrows - 1) / qrows, nblk_k = (a->Sk + 127) / 128;
  const int64_t Hkv = a->Hkv == 0 ? a->H : a->Hkv;
  if (Hkv < 0 || (a->H > 0 && (Hkv == 0 || a->H % Hkv != 0)) || (a->H == 0 && Hkv != 0))
    return fail(ATTN_E_INVALID, "H (%lld) must be a positive multiple of Hkv (%lld)",
                (long long)a->H, (long long)a->Hkv);
  if (a->H > 0 && a->B > INT32_MAX / a->H) return fail(ATTN_E_INVALID, "B * H too large");
  const int64_t heads = a->B * a->H;
  if (heads * (nblk_q > nblk_k ? nblk_q : nblk_k) > INT32_MAX)
    return fail(ATTN_E_INVALID, "problem too large for one launch");

  c.want_q = a->wrt == ATTN_WRT_Q || a->wrt == ATTN_WRT_ALL;
  c.want_k = a->wrt == ATTN_WRT_K || a->wrt == ATTN_WRT_ALL;
  c.want_v = a->wrt == ATTN_WRT_V || a->wrt == ATTN_WRT_ALL;
  c.bf16 = a->dtype == ATTN_BF16;
  c.D = (int)a->D;
  c.nblk_q = (int)nblk_q;
  c.nblk_k = (int)nblk_k;
  const size_t es = c.bf16 ? 2 : 4;
  const bool has_q = heads > 0 && a->Sq > 0, has_k = heads > 0 && a->Sk > 0;

  struct T {
    const char *name;
    const void *ptr;
    const int64_t *st;
    int64_t S, nh;  // sequence length, heads
    bool needed;
    bool output;
  } ts[7] = {
      {"q", a->q, a->q_stride, a->Sq, a->H, has_q, false},
      {"k", a->k, a->k_stride, a->Sk, Hkv, has_k, false},
      {"v", a->v, a->v_stride, a->Sk, Hkv, has_k, false},
      {"dy", a->dy, a->dy_stride, a->Sq, a->H, has_q, false},
      {"dq", a->dq, a->dq_stride, a->Sq, a->H, has_q && c.want_q, true},
      {"dk", a->dk, a->dk_stride, a->Sk, Hkv, has_k && c.want_k, true},
      {"dv", a->dv, a->dv_stride, a->Sk, Hkv, has_k && c.want_v, true},
  };
  Range rng[7];
  for (int i = 0; i < 7; ++i) {
    if (!ts[i].needed) continue;
    if (!ts[i].ptr) return fail(ATTN_E_INVALID, "%s is NULL", ts[i].name);
    for (int j = 0; j < 3; ++j)
      if (ts[i].st[j] < 0) return fail(ATTN_E_INVALID, "%s has a negative stride", ts[i].name);
    if ((uintptr_t)ts[i].ptr % 16)
      return fail(ATTN_E_UNSUPPORTED, "%s is not 16-byte aligned", ts[i].name);
    for (int j = 0; j < 3; ++j) {
      if (ts[i].st[j] > kMaxBytes)
        return fail(ATTN_E_INVALID, "%s stride %d is larger than 2^60", ts[i].name, j);
      if ((ts[i].st[j] * (int64_t)es) % 16)
        return fail(ATTN_E_UNSUPPORTED, "%s stride %d is not a multiple of 16 bytes", ts[i].name, j);
    }
    // Streamed chunks address their rows with 32-bit byte offsets.
    if (i < 4 && ts[i].st[1] * 64 * (int64_t)es >= ((int64_t)1 << 31))
      return fail(ATTN_E_UNSUPPORTED, "%s sequence stride %lld is too large (64 rows must span < 2 GiB)",
                  ts[i].name, (long long)ts[i].st[1]);
    const int64_t n[4] = {a->B, ts[i].S, ts[i].nh, a->D};
    const int64_t st[4] = {ts[i].st[0], ts[i].st[1], ts[i].st[2], 1};
    bool ok;
    rng[i] = extent(ts[i].ptr, n, st, es, ok);
    if (!ok) return fail(ATTN_E_INVALID, "%s spans more than 2^60 bytes", ts[i].name);
  }

  const bool masked = a->mask_kind == ATTN_MASK_KEYPAD || a->mask_kind == ATTN_MASK_BIAS;
  Range mrng;
  if (masked && has_q && a->Sk > 0) {
    if (!a->mask) return fail(ATTN_E_INVALID, "mask is NULL for mask_kind %d", a->mask_kind);
    if ((uintptr_t)a->mask % 4) return fail(ATTN_E_INVALID, "mask is not 4-byte aligned");
    for (int j = 0; j < 4; ++j)
      if (a->mask_stride[j] < 0) return fail(ATTN_E_INVALID, "mask has a negative stride");
    const int64_t n[4] = {a->B, a->H, a->Sq, a->Sk};
    bool ok;
    mrng = extent(a->mask, n, a->mask_stride, sizeof(float), ok);
    if (!ok) return fail(ATTN_E_INVALID, "mask spans more than 2^60 bytes");
  }

  const size_t ws_need = attn_bwd_workspace_bytes(a->B, a->H, a->Sq);
  Range wrng;
  c.ws_split = nullptr;
  if (ws_need) {
    if (!a->workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws_need);
    if ((uintptr_t)a->workspace % 256)
      return fail(ATTN_E_WORKSPACE, "workspace is not 256-byte aligned");
    if (a->workspace_bytes < ws_need)
      return fail(ATTN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", a->workspace_bytes, ws_need);
    wrng.lo = (uintptr_t)a->workspace;
    wrng.hi = wrng.lo + ws_need;
    // a workspace of attn_bwd_split_workspace_bytes() enables the split form
    const size_t split_need = attn_bwd_split_workspace_bytes(a->B, a->H, a->Sq, a->Sk, a->D);
    if (split_need > ws_need && a->workspace_bytes >= split_need) {
      c.ws_split = (float *)((char *)a->workspace + ws_need);
      wrng.hi = wrng.lo + split_need;
    }
  }

  // No output may share memory with an input, another output or the workspace.
  for (int i = 4; i < 7; ++i) {
    if (!ts[i].needed) continue;
    for (int j = 0; j < 7; ++j)
      if (j != i && ts[j].needed && overlap(rng[i], rng[j]))
        return fail(ATTN_E_INVALID, "%s overlaps %s", ts[i].name, ts[j].name);
    if (overlap(rng[i], mrng)) return fail(ATTN_E_INVALID, "%s overlaps mask", ts[i].name);
    if (overlap(rng[i], wrng)) return fail(ATTN_E_INVALID, "%s overlaps the workspace", ts[i].name);
  }
  if (overlap(wrng, mrng)) return fail(ATTN_E_INVALID, "workspace overlaps mask");
  for (int j = 0; j < 4; ++j)
    if (ts[j].needed && overlap(wrng, rng[j]))
      return fail(ATTN_E_INVALID, "workspace overlaps %s", ts[j].name);

  attn::DenseParams &p = c.p;
  std::memset(&p, 0, sizeof p);
  p.q = a->q; p.k = a->k; p.v = a->v; p.dy = a->dy;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  for (int j = 0; j < 3; ++j) {
    p.qs[j] = a->q_stride[j]; p.ks[j] = a->k_stride[j]; p.vs[j] = a->v_stride[j];
    p.dys[j] = a->dy_stride[j]; p.dqs[j] = a->dq_stride[j]; p.dks[j] = a->dk_stride[j];
    p.dvs[j] = a->dv_stride[j];
  }
  p.mask = masked ? a->mask : nullptr;
  for (int j = 0; j < 4; ++j) p.ms[j] = masked ? a->mask_stride[j] : 0;
  p.thr = a->mask_threshold;
  p.scale = a->scale;
  p.scale_log2 = a->scale * attn::kLog2e;
  p.inv_scale_log2 = 1.f / p.scale_log2;
  p.B = (int)a->B; p.H = (int)a->H; p.Sq = (int)a->Sq; p.Sk = (int)a->Sk;
  p.Hkv = (int)Hkv;
  p.G = Hkv > 0 ? (int)(a->H / Hkv) : 1;
  // Query i sits at absolute position max(Sk - Sq, 0) + i (rlx-cpu
  // `apply_synthetic_mask`, saturating_sub).
  const int64_t q_off = a->Sk > a->Sq ? a->Sk - a->Sq : 0;
  const bool causal = a->mask_kind == ATTN_MASK_CAUSAL || a->mask_kind == ATTN_MASK_WINDOW ||
                      (a->mask_flags & ATTN_MASK_FLAG_CAUSAL);
  p.hi_off = causal ? (int)q_off : attn::kBig;
  if (a->mask_kind == ATTN_MASK_WINDOW) {
    const int64_t lo = q_off - a->window;
    p.lo_off = lo < -(int64_t)attn::kBig ? -attn::kBig : (int)lo;
  } else {
    p.lo_off = -attn::kBig;
  }
  p.need_dk = c.want_k;
  p.need_dv = c.want_v;
  char *ws = (char *)a->workspace;
  const size_t pb = plane_bytes(a->B, a->H, a->Sq);
  p.st_m = (float *)ws;
  p.st_l = (float *)(ws ? ws + pb : nullptr);
  p.st_delta = (float *)(ws ? ws + 2 * pb : nullptr);
  p.st_nls = (float *)(ws ? ws + 3 * pb : nullptr);
  c.mode = a->mask_kind == ATTN_MASK_KEYPAD ? attn::MODE_KEYPAD
           : a->mask_kind == ATTN_MASK_BIAS ? attn::MODE_BIAS
                                            : attn::MODE_INDEX;
  return ATTN_OK;
}

int run_stage(int stage, Checked &c, hipStream_t stream) {
  attn::DenseParams p = c.p;
  const int heads = p.B * p.H;
  int nblocks = 0;
  if (stage == attn::STAGE_ROW_STATS) {
    if (p.Sq == 0 || !(c.want_q || c.want_k || c.want_v)) return ATTN_OK;
    p.nblk = c.nblk_q;
    nblocks = heads * c.nblk_q;
  } else if (stage == attn::STAGE_KV) {
    if (!(c.want_k || c.want_v) || p.Sk == 0) return ATTN_OK;
    p.nblk = c.nblk_k;
    nblocks = p.B * p.Hkv * c.nblk_k;  // one key block of one K / V head each
  } else if (stage == attn::STAGE_DQ) {
    if (!c.want_q || p.Sq == 0) return ATTN_OK;
    p.nblk = c.nblk_q;
    nblocks = heads * c.nblk_q;
  } else {  // STAGE_STATS_DQ (bf16): statistics always, dQ if asked
    if (p.Sq == 0 || !(c.want_q || c.want_k || c.want_v)) return ATTN_OK;
    if (!c.want_q) p.dq = nullptr;
    p.nblk = c.nblk_q;
    nblocks = heads * c.nblk_q;
  }
  // Split form: not for the dQ pass that forms a forward's statistics (it also
  // publishes them).
  if (c.ws_split && !(stage == attn::STAGE_DQ && p.fo)) {
    const bool kv = stage == attn::STAGE_KV;
    const int unit = kv ? (c.bf16 ? 64 : 32) : stage == attn::STAGE_STATS_DQ ? 64 : 32;  // chunk rows
    const int64_t n = kv ? p.Sq : p.Sk;
    const int np = split_pieces(nblocks, split_max_pieces(n, unit), attn::device_cus());
    if (np >= 2) {
      const int chunks = (int)((n + unit - 1) / unit);
      p.piece_chunks = (chunks + np - 1) / np;
      p.npiece = (chunks + p.piece_chunks - 1) / p.piece_chunks;  // no empty tail piece
      p.ws_split = c.ws_split;
    }
  }
  const hipError_t e = attn::launch_dense_stage(stage, c.bf16, c.D, c.mode, p, nblocks, stream);
  if (e != hipSuccess)
    return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int run(const attn_bwd_args *a, void *stream, int first, int last) {
  Checked c;
  const int rc = validate(a, c);
  if (rc != ATTN_OK) return rc;
  for (int s = first; s <= last; ++s) {
    const int r = run_stage(s, c, (hipStream_t)stream);
    if (r != ATTN_OK) return r;
  }
  return ATTN_OK;
}

// Dense backward from a forward's saved statistics: lse and O replace the row
// statistics pass.
int run_from_forward(const attn_bwd_args *a, const float *lse, const void *out,
                     const int64_t *out_stride, void *stream) {
  Checked c;
  int rc = validate(a, c);
  if (rc != ATTN_OK) return rc;
  const int64_t rows = a->B * a->H * a->Sq;
  const bool any = rows > 0 && a->Sk > 0 && (c.want_q || c.want_k || c.want_v);
  if (any) {
    if (!lse || !out || !out_stride) return fail(ATTN_E_INVALID, "lse / out / out_stride is NULL");
    const size_t es = c.bf16 ? 2 : 4;
    if ((uintptr_t)lse % 4) return fail(ATTN_E_INVALID, "lse is not 4-byte aligned");
    if ((uintptr_t)out % 16) return fail(ATTN_E_UNSUPPORTED, "out is not 16-byte aligned");
    for (int j = 0; j < 3; ++j) {
      if (out_stride[j] < 0) return fail(ATTN_E_INVALID, "out has a negative stride");
      if (out_stride[j] > kMaxBytes) return fail(ATTN_E_INVALID, "out stride %d is larger than 2^60", j);
      if ((out_stride[j] * (int64_t)es) % 16)
        return fail(ATTN_E_UNSUPPORTED, "out stride %d is not a multiple of 16 bytes", j);
    }
    // The workspace planes written here must not alias the inputs read.
    Range ws, lr, orng;
    ws.lo = (uintptr_t)a->workspace;
    ws.hi = ws.lo + attn_bwd_workspace_bytes(a->B, a->H, a->Sq);
    lr.lo = (uintptr_t)lse;
    lr.hi = lr.lo + (uintptr_t)(rows * 4);
    const int64_t n[4] = {a->B, a->Sq, a->H, a->D};
    const int64_t st[4] = {out_stride[0], out_stride[1], out_stride[2], 1};
    bool ok;
    orng = extent(out, n, st, es, ok);
    if (!ok) return fail(ATTN_E_INVALID, "out spans more than 2^60 bytes");
    if (overlap(ws, lr) || overlap(ws, orng))
      return fail(ATTN_E_INVALID, "lse / out overlap the workspace");
    // The dQ kernel forms delta and -lse2 from lse and O in its prologue and
    // publishes them (without dQ asked for it stops there); the dK / dV kernel
    // follows it on the stream.  Every `wrt` takes the same statistics.
    Checked cq = c;
    cq.p.fo = out;
    cq.p.flse = lse;
    for (int j = 0; j < 3; ++j) cq.p.fos[j] = out_stride[j];
    if (!c.want_q) {
      cq.want_q = true;
      cq.p.dq = nullptr;
    }
    rc = run_stage(attn::STAGE_DQ, cq, (hipStream_t)stream);
    if (rc != ATTN_OK) return rc;
    return run_stage(attn::STAGE_KV, c, (hipStream_t)stream);
  }
  // Nothing to read (no rows or no keys): the stages write their zeros.
  for (int s = attn::STAGE_KV; s <= attn::STAGE_DQ; ++s) {
    rc = run_stage(s, c, (hipStream_t)stream);
    if (rc != ATTN_OK) return rc;
  }
  return ATTN_OK;
}

// ---------------------------------------------------------------------------
// Paged history backward.

// What a paged call computes: dK / dV (attn_bwd_paged), the statistics, dQ or
// both (the query side).  PM_SDQ: out = the statistics, out2 = dQ.
enum PagedMode { PM_KV = 0, PM_STATS = 1, PM_DQ = 2, PM_SDQ = 3 };

int validate_paged(const attn_bwd_paged_args *a, int mode, void *out, void *out2,
                   attn::PagedParams &p, int &nblocks, bool &bf16) {
  using namespace attn::plan;
  if (!a) return fail(ATTN_E_INVALID, "args is NULL");
  if (a->dtype != ATTN_F32 && a->dtype != ATTN_BF16)
    return fail(ATTN_E_INVALID, "dtype %d is not ATTN_F32 or ATTN_BF16", a->dtype);
  if (a->mla != 0 && a->mla != 1) return fail(ATTN_E_INVALID, "mla must be 0 or 1");
  const bool mla = a->mla == 1;
  if (mla && mode != PM_KV)
    return fail(ATTN_E_UNSUPPORTED, "the query side does not take the latent variant");
  if (mode == PM_KV && !mla && (a->need < 1 || a->need > 3))
    return fail(ATTN_E_INVALID, "need %d is not 1, 2 or 3", a->need);
  if (mode == PM_KV && mla && (a->need < 1 || a->need > 5 || (a->need & 2)))
    return fail(ATTN_E_INVALID, "latent variant: need %d is not 1, 4 or 5", a->need);
  if (mla) {
    const bool wide = a->dtype == ATTN_BF16 && (a->head_dim == 192 || a->head_dim == 256);
    if (a->head_dim != 64 && a->head_dim != 128 && !wide)
      return fail(ATTN_E_UNSUPPORTED,
                  "latent width %d is not 64 or 128 (or, for bf16, 192 or 256)", a->head_dim);
    if (a->position_dim != 0 && a->position_dim != 32 && a->position_dim != 64)
      return fail(ATTN_E_UNSUPPORTED, "position_dim %d is not 0, 32 or 64", a->position_dim);
    if ((a->need & 4) && a->position_dim == 0)
      return fail(ATTN_E_INVALID, "need asks for position-key gradients but position_dim is 0");
  } else if (a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128) {
    return fail(ATTN_E_UNSUPPORTED, "head_dim %d is not 32, 64 or 128", a->head_dim);
  }
  if (!std::isfinite(a->scale)) return fail(ATTN_E_INVALID, "scale is not finite");
  if (std::fabs(a->scale) < kMinScale || std::fabs(a->scale) > kMaxScale)
    return fail(ATTN_E_UNSUPPORTED, "|scale| outside [2^-64, 2^64] (including 0) is not supported");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1");
  if (a->kv_workgroups < -1) return fail(ATTN_E_INVALID, "kv_workgroups is below -1");
  if (mode == PM_SDQ && (a->q_form < 0 || a->q_form > 2))
    return fail(ATTN_E_INVALID, "q_form %d is not 0, 1 or 2", a->q_form);
  const int32_t *w = a->plan_host;
  if (!w || !a->plan) return fail(ATTN_E_INVALID, "plan_host / plan is NULL");
  if (w[W_MAGIC] != kMagic) return fail(ATTN_E_INVALID, "plan_host is not a plan (bad magic)");
  const int64_t words = w[W_WORDS];
  if (words < HEADER_WORDS) return fail(ATTN_E_INVALID, "plan header is inconsistent");
  for (int k = W_OFF_ITEM_LINKS; k <= W_OFF_QPIECE_ORDER; ++k) {
    if (k == W_TOKENS || k == W_QBLK) continue;
    if (w[k] < HEADER_WORDS || w[k] > words) return fail(ATTN_E_INVALID, "plan offsets are inconsistent");
  }
  if (w[W_HEADS] != a->heads || w[W_KV_HEADS] != a->kv_heads || w[W_PAGE_SIZE] != a->page_size ||
      w[W_NQ] != a->nq || w[W_POOL_PAGES] != a->pool_pages)
    return fail(ATTN_E_INVALID,
                "plan was built for heads %d, kv_heads %d, page_size %d, nq %d, pool_pages %d",
                w[W_HEADS], w[W_KV_HEADS], w[W_PAGE_SIZE], w[W_NQ], w[W_POOL_PAGES]);
  const int64_t items = w[W_ITEMS], qblocks = w[W_QBLK], qpieces = w[W_QPIECES];
  if (items < 0 || items * (int64_t)a->kv_heads > INT32_MAX || qblocks < 0 ||
      qblocks * (int64_t)a->kv_heads > INT32_MAX || qpieces < 0 ||
      qpieces * (int64_t)a->kv_heads > INT32_MAX ||
      qblocks * (int64_t)a->kv_heads * attn::kQBlockRows * 32 > INT32_MAX * (int64_t)256)
    return fail(ATTN_E_INVALID, "plan item count is inconsistent");
  bf16 = a->dtype == ATTN_BF16;
  nblocks = (int)((mode == PM_KV ? items : qblocks) * a->kv_heads);

  const size_t es = bf16 ? 2 : 4;
  const int64_t D = a->head_dim, P = mla ? a->position_dim : 0;
  const int64_t qrows = (int64_t)a->nq * a->heads;
  const int64_t pslots = (int64_t)a->pool_pages * a->page_size * a->kv_heads;
  const bool work = nblocks > 0, kv = mode == PM_KV;
  constexpr int NT = 12, FIRST_OUT = 8;
  const bool st_out = mode == PM_STATS || mode == PM_SDQ;
  struct T {
    const char *name;
    const void *ptr;
    int64_t bytes;
    bool needed;
  } ts[NT] = {
      {"q", a->q, qrows * D * (int64_t)es, work && qrows > 0},
      {"dy", a->dy, qrows * D * (int64_t)es, work && qrows > 0},
      {"stats", a->stats, qrows * 3 * (int64_t)sizeof(float), work && qrows > 0 && (mode == PM_KV || mode == PM_DQ)},
      {"k_pool", a->k_pool, pslots * D * (int64_t)es, work},
      {"v_pool", a->v_pool, pslots * D * (int64_t)es, work && !mla},
      {"qp", a->qp, qrows * P * (int64_t)es, work && qrows > 0 && P > 0},
      {"kp_pool", a->kp_pool, pslots * P * (int64_t)es, work && P > 0},
      {"plan", a->plan, (int64_t)words * 4, work},
      {"dk_pool", a->dk_pool, pslots * D * (int64_t)es, work && kv && (a->need & 1)},
      {"dv_pool", a->dv_pool, pslots * D * (int64_t)es, work && kv && !mla && (a->need & 2)},
      {kv ? "dkp_pool" : (st_out ? "stats_out" : "dq"), kv ? a->dkp_pool : out,
       kv ? pslots * P * (int64_t)es
          : qrows * (st_out ? 3 * (int64_t)sizeof(float) : D * (int64_t)es),
       work && (kv ? mla && (a->need & 4) : true)},
      {"dq", out2, qrows * D * (int64_t)es, work && mode == PM_SDQ},
  };
  Range rng[NT];
  for (int i = 0; i < NT; ++i) {
    if (!ts[i].needed) continue;
    if (!ts[i].ptr) return fail(ATTN_E_INVALID, "%s is NULL", ts[i].name);
    const unsigned align = i == 7 ? 4 : 16;  // the plan is read as int32 words
    if ((uintptr_t)ts[i].ptr % align)
      return fail(ATTN_E_UNSUPPORTED, "%s is not %u-byte aligned", ts[i].name, align);
    rng[i].lo = (uintptr_t)ts[i].ptr;
    rng[i].hi = rng[i].lo + (uintptr_t)ts[i].bytes;
  }
  for (int i = FIRST_OUT; i < NT; ++i) {  // outputs
    if (!ts[i].needed) continue;
    for (int j = 0; j < NT; ++j)
      if (j != i && ts[j].needed && overlap(rng[i], rng[j]))
        return fail(ATTN_E_INVALID, "%s overlaps %s", ts[i].name, ts[j].name);
  }

  // Query side, split form: the partial results' workspace.
  float *qws = nullptr;
  if (mode != PM_KV && a->q_workspace && work) {
    const int64_t need = qpieces * a->kv_heads * attn::kQBlockRows *
                         (mode == PM_STATS ? 4 : mode == PM_SDQ && bf16 ? 2 * D + 8 : D) *
                         (int64_t)sizeof(float);
    if ((int64_t)a->q_workspace_bytes < need)
      return fail(ATTN_E_WORKSPACE, "q_workspace_bytes %zu < %lld needed", a->q_workspace_bytes,
                  (long long)need);
    if ((uintptr_t)a->q_workspace % 16)
      return fail(ATTN_E_UNSUPPORTED, "q_workspace is not 16-byte aligned");
    Range wr;
    wr.lo = (uintptr_t)a->q_workspace;
    wr.hi = wr.lo + (uintptr_t)need;
    for (int j = 0; j < NT; ++j)
      if (ts[j].needed && overlap(wr, rng[j]))
        return fail(ATTN_E_INVALID, "q_workspace overlaps %s", ts[j].name);
    qws = (float *)a->q_workspace;
  }

  std::memset(&p, 0, sizeof p);
  p.qws = qws;
  p.off_qpiece = w[W_OFF_QPIECE];
  p.off_qblk_piece = w[W_OFF_QBLK_PIECE];
  p.off_qpiece_order = w[W_OFF_QPIECE_ORDER];
  p.qpieces = (int)qpieces;
  p.q = a->q; p.dy = a->dy; p.k_pool = a->k_pool; p.v_pool = a->v_pool;
  p.dk_pool = a->dk_pool; p.dv_pool = a->dv_pool;
  if (mla) {
    p.mla = 1;
    p.P = (int)P;
    p.qp = a->qp;
    p.kp_pool = a->kp_pool;
    p.dkp_pool = a->dkp_pool;
    p.need_dkp = (a->need >> 2) & 1;
  }
  if (mode == PM_STATS || mode == PM_SDQ) p.stats_out = (float *)out;
  if (mode == PM_DQ) p.dq = out;
  if (mode == PM_SDQ) p.dq = out2;
  p.stats = a->stats;
  p.plan = a->plan;
  p.heads = a->heads;
  p.kv_heads = a->kv_heads;
  p.group = a->heads / a->kv_heads;
  p.causal = a->causal;
  p.need_dk = a->need & 1;
  p.need_dv = mla ? 0 : (a->need >> 1) & 1;
  p.scale = a->scale;
  p.scale_log2 = a->scale * attn::kLog2e;
  p.inv_scale_log2 = 1.f / p.scale_log2;
  p.items = (int)items;
  p.off_item_links = w[W_OFF_ITEM_LINKS];
  p.off_item_slots = w[W_OFF_ITEM_SLOTS];
  p.off_link_seq = w[W_OFF_LINK_SEQ];
  p.off_link_info = w[W_OFF_LINK_INFO];
  p.off_link_tok = w[W_OFF_LINK_TOK];
  p.off_seq_qh = w[W_OFF_SEQ_QH];
  p.off_qh_rh = w[W_OFF_QH_RH];
  p.off_qh_pos = w[W_OFF_QH_POS];
  p.off_seq_maxpos = w[W_OFF_SEQ_MAXPOS];
  p.off_seq_minpos = w[W_OFF_SEQ_MINPOS];
  p.off_seq_tok = w[W_OFF_SEQ_TOK];
  p.off_tok_slot = w[W_OFF_TOK_SLOT];
  p.off_qblk = w[W_OFF_QBLK];
  p.qblocks = w[W_QBLK];
  return ATTN_OK;
}

}  // namespace

namespace attn {
void set_last_error(const char *msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
}
hipError_t launch_paged(bool bf16_in, int D, const PagedParams &p, int nblocks, int workgroups,
                        hipStream_t stream);
hipError_t launch_paged_q(int stage, bool bf16_in, int D, const PagedParams &p, int nblocks,
                          hipStream_t stream);
int device_cus();
}  // namespace attn

namespace {
// The fused query pass (bf16) with a workspace: whether the split form's
// estimated time is below the direct form's, from the host plan, in units of
// one 64-token chunk step of one workgroup (one workgroup per compute unit).
// A unit (a query block or a piece of one, per KV head) costs its visible
// chunks plus kFixed steps (loading its rows and first chunks, storing its
// results); a form takes at least its longest unit and its total over the
// compute units; the split form adds one longest piece for the rounds'
// granularity and the merge's traffic (each piece's partial results written
// and read once).
bool sdq_split_is_faster(const int32_t *w, int kv_heads, int causal, int D, int cus) {
  using namespace attn::plan;
  constexpr double kFixed = 5.0, kStepBytes = 7.6e6;  // HBM bytes moved per step time
  const int64_t words = w[W_WORDS], nseq = w[W_NSEQ], nb = w[W_QBLK], np = w[W_QPIECES];
  const int64_t ob = w[W_OFF_QBLK], otok = w[W_OFF_SEQ_TOK], omax = w[W_OFF_SEQ_MAXPOS];
  const int64_t opc = w[W_OFF_QPIECE];
  if (cus <= 0 || nseq < 0 || ob + 2 * nb > words || otok + nseq + 1 > words ||
      omax + nseq > words || opc + 3 * np > words)
    return false;
  auto visible = [&](int64_t b) -> int64_t {  // tokens the block's rows see, -1 for a bad entry
    if (b < 0 || b >= nb) return -1;
    const int64_t s = w[ob + 2 * b];
    if (s < 0 || s >= nseq) return -1;
    const int64_t len = (int64_t)w[otok + s + 1] - w[otok + s];
    return causal ? std::min<int64_t>(len, (int64_t)w[omax + s] + 1) : len;
  };
  auto chunks = [](int64_t t) { return t > 0 ? (double)((t + 63) / 64) : 0.0; };
  double dmax = 0, dsum = 0, smax = 0, ssum = 0;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t v = visible(b);
    if (v < 0) return false;
    const double c = chunks(v) + kFixed;
    dmax = std::max(dmax, c);
    dsum += c;
  }
  for (int64_t k = 0; k < np; ++k) {
    const int64_t v = visible(w[opc + 3 * k]);
    if (v < 0) return false;
    const double c = chunks(std::min<int64_t>(w[opc + 3 * k + 2], v) - w[opc + 3 * k + 1]) + kFixed;
    smax = std::max(smax, c);
    ssum += c;
  }
  const double direct = std::max(dmax, dsum * kv_heads / cus);
  const double merge = 2.0 * np * kv_heads * attn::kQBlockRows * (2.0 * D + 8) * 4 / kStepBytes;
  const double split = std::max(smax, ssum * kv_heads / cus) + smax + merge;
  return split < direct;
}

int run_paged(const attn_bwd_paged_args *a, int mode, void *out, void *out2, void *stream) {
  attn::PagedParams p;
  int nblocks = 0;
  bool bf16 = false;
  const int rc = validate_paged(a, mode, out, out2, p, nblocks, bf16);
  if (rc != ATTN_OK) return rc;
  if (mode == PM_SDQ && bf16) {
    if (a->q_form == 1 && !p.qws)
      return fail(ATTN_E_WORKSPACE, "q_form 1 (split) needs q_workspace");
    if (a->q_form == 2 ||
        (a->q_form == 0 && p.qws &&
         !sdq_split_is_faster(a->plan_host, a->kv_heads, a->causal, a->head_dim,
                              attn::device_cus())))
      p.qws = nullptr;  // the direct form
  }
  if (nblocks == 0) return ATTN_OK;
  const hipError_t e =
      mode == PM_KV ? attn::launch_paged(bf16, a->head_dim, p, nblocks, a->kv_workgroups,
                                         (hipStream_t)stream)
                    : attn::launch_paged_q(mode == PM_STATS ? 0 : mode == PM_DQ ? 1 : 2, bf16,
                                           a->head_dim, p, nblocks, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}
}  // namespace

extern "C" {

int attn_bwd_paged(const attn_bwd_paged_args *a, void *stream) {
  return run_paged(a, PM_KV, nullptr, nullptr, stream);
}

int attn_bwd_paged_row_stats(const attn_bwd_paged_args *a, float *stats, void *stream) {
  return run_paged(a, PM_STATS, stats, nullptr, stream);
}

int attn_bwd_paged_dq(const attn_bwd_paged_args *a, void *dq, void *stream) {
  return run_paged(a, PM_DQ, dq, nullptr, stream);
}

int attn_bwd_paged_stats_dq(const attn_bwd_paged_args *a, float *stats, void *dq, void *stream) {
  return run_paged(a, PM_SDQ, stats, dq, stream);
}

size_t attn_bwd_paged_q_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace attn::plan;
  if (!plan_host || plan_host[W_MAGIC] != kMagic || head_dim <= 0 || plan_host[W_QPIECES] < 0 ||
      plan_host[W_KV_HEADS] <= 0) {
    fail(ATTN_E_INVALID, "not a plan, or head_dim <= 0");
    return 0;
  }
  return (size_t)plan_host[W_QPIECES] * (size_t)plan_host[W_KV_HEADS] * attn::kQBlockRows *
         (2 * (size_t)head_dim + 8) * sizeof(float);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq) {
  if (B < 0 || H < 0 || Sq < 0) return 0;
  if (stat_bytes(B, H, Sq) < 0) return SIZE_MAX;  // never satisfiable
  return 4 * plane_bytes(B, H, Sq);
}

size_t attn_bwd_split_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0 || D > 4096) return 0;
  const size_t base = attn_bwd_workspace_bytes(B, H, Sq);
  if (base == SIZE_MAX) return base;
  // query-major passes: pieces of the keys, max(D, 4) floats per query row
  // (the fused bf16 pass: pieces of 64 keys, 2 D + 8); dK / dV: pieces of the
  // queries, 2 D floats per key row (H bounds Hkv)
  const int64_t npq = split_max_pieces(Sk), npf = split_max_pieces(Sk, 64),
                npk = split_max_pieces(Sq);
  const int64_t rq = stat_bytes(B, H, Sq), rk = stat_bytes(B, H, Sk);
  int64_t nq = 0, nf = 0, nk = 0;
  if (rq < 0 || rk < 0 || __builtin_mul_overflow(rq, npq * (D > 4 ? D : 4), &nq) ||
      __builtin_mul_overflow(rq, npf * (2 * D + 8), &nf) ||
      __builtin_mul_overflow(rk, npk * 2 * D, &nk) || nq > kMaxBytes || nf > kMaxBytes ||
      nk > kMaxBytes)
    return base;
  const int64_t n = std::max({npq >= 2 ? nq : 0, npf >= 2 ? nf : 0, npk >= 2 ? nk : 0});
  return base + (size_t)n;
}

}  // extern "C"

// bf16: one query-major pass for the statistics and dQ, then dK / dV.
// fp32: statistics, dK / dV, dQ (three passes; dQ from the exact delta).
// Also the body of attn_bwd_noalloc (noalloc.hip), with its workspace filled in.
int attn::run_dense_all(const attn_bwd_args *a, void *stream) {
  Checked c;
  const int rc = validate(a, c);
  if (rc != ATTN_OK) return rc;
  static const int bf16_order[] = {attn::STAGE_STATS_DQ, attn::STAGE_KV};
  static const int f32_order[] = {attn::STAGE_ROW_STATS, attn::STAGE_KV, attn::STAGE_DQ};
  const int *order = c.bf16 ? bf16_order : f32_order;
  const int n = c.bf16 ? 2 : 3;
  for (int i = 0; i < n; ++i) {
    const int r = run_stage(order[i], c, (hipStream_t)stream);
    if (r != ATTN_OK) return r;
  }
  return ATTN_OK;
}

extern "C" {

int attn_bwd(const attn_bwd_args *a, void *stream) { return attn::run_dense_all(a, stream); }



int attn_bwd_stats_dq(const attn_bwd_args *a, void *stream) {
  Checked c;
  const int rc = validate(a, c);
  if (rc != ATTN_OK) return rc;
  if (c.bf16) return run_stage(attn::STAGE_STATS_DQ, c, (hipStream_t)stream);
  const int r = run_stage(attn::STAGE_ROW_STATS, c, (hipStream_t)stream);
  return r != ATTN_OK ? r : run_stage(attn::STAGE_DQ, c, (hipStream_t)stream);
}

int attn_bwd_row_stats(const attn_bwd_args *a, void *stream) {
  return run(a, stream, attn::STAGE_ROW_STATS, attn::STAGE_ROW_STATS);
}

int attn_bwd_kv(const attn_bwd_args *a, void *stream) {
  return run(a, stream, attn::STAGE_KV, attn::STAGE_KV);
}

int attn_bwd_from_forward(const attn_bwd_args *a, const float *lse, const void *out,
                          const int64_t *out_stride, void *stream) {
  return run_from_forward(a, lse, out, out_stride, stream);
}

int attn_bwd_dq(const attn_bwd_args *a, void *stream) {
  return run(a, stream, attn::STAGE_DQ, attn::STAGE_DQ);
}

const char *attn_bwd_last_error(void) { return g_err; }

}  // extern "C"
