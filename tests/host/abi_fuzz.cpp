// abi_fuzz.cpp -- host-only stress driver of the library's C ABI validation
// (abi.cpp) and paged planner (paged_plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU is involved: the kernel launchers are
// replaced by stubs that check what the validated parameters promise the
// kernels (grid sizes, geometry, plan tables inside the plan), and every
// device pointer handed to the ABI is a fake address that is never touched.
//
// A seeded sweep draws valid and malformed arguments: sizes from 0 to 2^63,
// negative and huge strides, NULL and misaligned pointers, overlapping
// tensors, NaN / zero / infinite scales and thresholds, every enum value and
// some that are not; block tables with shared, repeated and out-of-range
// pages, query rows out of range, plans with corrupted header offsets.  Each
// call must return a defined status (with a message when it is not ATTN_OK);
// the sanitizers turn any out-of-bounds access, overflow or invalid shift in
// the host code into a failure.
//
// Usage: abi_fuzz <iterations> <seed>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "attn_bwd.h"
#include "launch.hpp"
#include "paged.hpp"

namespace {

std::mt19937_64 rng;
long n_launch = 0;

[[noreturn]] void die(const char *what) {
  std::fprintf(stderr, "abi_fuzz: invariant broken: %s\n", what);
  std::abort();
}

int64_t pick(std::initializer_list<int64_t> v) {
  return *(v.begin() + rng() % v.size());
}
bool chance(int percent) { return (int)(rng() % 100) < percent; }
int64_t small(int64_t hi) { return (int64_t)(rng() % (uint64_t)(hi + 1)); }

// a * b, saturated to int64 range (the fuzzer itself must stay free of overflow).
int64_t smul(int64_t a, int64_t b) {
  __int128 r = (__int128)a * b;
  if (r > INT64_MAX) return INT64_MAX;
  if (r < INT64_MIN) return INT64_MIN;
  return (int64_t)r;
}

// A fake device address: 256-aligned in [2^32, 2^44), sometimes misaligned or NULL.
uintptr_t fake_ptr() {
  if (chance(3)) return 0;
  uintptr_t p = ((uintptr_t)1 << 32) + ((rng() % ((uint64_t)1 << 36)) << 8);
  if (chance(3)) p += pick({4, 8, 2});
  return p;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launcher stubs: what every accepted call hands the kernels.
namespace attn {

hipError_t launch_dense_stage(int stage, bool bf16, int D, int mode, const DenseParams &p, int nblocks,
                              hipStream_t) {
  ++n_launch;
  if (stage < STAGE_ROW_STATS || stage > STAGE_STATS_DQ) die("dense stage");
  if (nblocks < 0) die("dense grid");
  if (nblocks == 0) return hipSuccess;  // the real launcher enqueues nothing either
  if (D != 32 && D != 64 && D != 128) die("dense head_dim");
  if (mode < MODE_INDEX || mode > MODE_BIAS) die("dense mask mode");
  if (p.B < 0 || p.H < 0 || p.Sq < 0 || p.Sk < 0 || p.Sq >= (1 << 30) || p.Sk >= (1 << 30))
    die("dense sizes");
  if (p.Hkv < 1 || p.G < 1 || (int64_t)p.Hkv * p.G != p.H) die("dense head groups");
  if (!(std::isfinite(p.scale) && std::isfinite(p.scale_log2) && std::isfinite(p.inv_scale_log2)))
    die("dense scale");
  if (p.nblk < 1) die("dense blocks per head");
  const int64_t heads = (int64_t)p.B * (stage == STAGE_KV ? p.Hkv : p.H);
  if ((int64_t)nblocks != heads * p.nblk) die("dense grid size");
  if (!p.st_m || !p.st_l || !p.st_delta || !p.st_nls) die("dense workspace planes");
  if ((mode != MODE_INDEX) != (p.mask != nullptr)) die("dense mask pointer");
  if (p.ws_split) {  // split form: pieces covering the streamed axis
    if (stage == STAGE_DQ && p.fo) die("split dQ pass with a forward's statistics");
    if (p.npiece < 2 || p.npiece > 16 || p.piece_chunks < 4) die("split pieces");
    const int64_t unit = stage == STAGE_KV ? (bf16 ? 64 : 32) : stage == STAGE_STATS_DQ ? 64 : 32;
    const int64_t n = stage == STAGE_KV ? p.Sq : p.Sk;
    const int64_t chunks = (n + unit - 1) / unit;
    if ((int64_t)p.npiece * p.piece_chunks < chunks || (int64_t)(p.npiece - 1) * p.piece_chunks >= chunks)
      die("split pieces do not tile the keys");
    if ((char *)p.ws_split < (char *)p.st_nls) die("split region below the planes");
  }
  return hipSuccess;
}

hipError_t launch_paged(bool bf16, int D, const PagedParams &p, int nblocks, int workgroups,
                        hipStream_t) {
  ++n_launch;
  if (workgroups < -1) die("paged kv_workgroups below -1 reached the launcher");
  if (nblocks <= 0 || (int64_t)nblocks != (int64_t)p.items * p.kv_heads) die("paged grid");
  if (p.mla ? (D != 64 && D != 128 && !(bf16 && (D == 192 || D == 256)))
            : (D != 32 && D != 64 && D != 128))
    die("paged head_dim");
  if (p.group < 1 || p.group * p.kv_heads != p.heads) die("paged group");
  if (!p.plan) die("paged plan pointer");
  return hipSuccess;
}

int device_cus() { return 256; }  // the split decisions see a 256-CU device

hipError_t launch_paged_q(int stage, bool, int D, const PagedParams &p, int nblocks, hipStream_t) {
  ++n_launch;
  if (stage != 0 && stage != 1 && stage != 2) die("paged query stage");
  if (stage == 2 && (!p.stats_out || !p.dq)) die("paged fused outputs");
  if (nblocks <= 0 || (int64_t)nblocks != (int64_t)p.qblocks * p.kv_heads) die("paged query grid");
  if (D != 32 && D != 64 && D != 128) die("paged query head_dim");
  if (p.qws && p.qpieces < 0) die("paged query pieces");
  return hipSuccess;
}

}  // namespace attn

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

namespace {

void check_status(int rc, const char *entry) {
  if (rc != ATTN_OK && rc != ATTN_E_INVALID && rc != ATTN_E_UNSUPPORTED && rc != ATTN_E_WORKSPACE &&
      rc != ATTN_E_HIP)
    die(entry);
  if (rc != ATTN_OK && attn_bwd_last_error()[0] == '\0') die("a rejection without a message");
}

// ---------------------------------------------------------------------------
// Dense entry points.

int64_t dim() {
  if (chance(70)) return pick({0, 1, 2, 3, 5, 16, 64, 127, 128, 129, 1000, 2048});
  return pick({(1 << 30) - 1, 1 << 30, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX, INT64_MIN,
               -1, -5, INT32_MAX});
}

void contiguous(int64_t S, int64_t H, int64_t D, int64_t st[3]) {
  st[2] = D;
  st[1] = smul(H, D);
  st[0] = smul(S, st[1]);
}

void fill_strides(int64_t S, int64_t H, int64_t D, int64_t st[3]) {
  contiguous(S, H, D, st);
  if (chance(15)) {  // [B, H, S, D]
    st[1] = D;
    st[2] = smul(S, D);
    st[0] = smul(H, st[2]);
  }
  if (chance(10)) st[rng() % 3] = pick({-1, -16, 0, 7, INT64_MAX, INT64_MIN, (int64_t)1 << 40});
}

// A well-formed dense call: small sizes, non-overlapping fake tensors 2^40
// bytes apart, contiguous or [B, H, S, D] strides; then, sometimes, one field
// replaced by a boundary value.
void make_valid(attn_bwd_args &a) {
  a.dtype = (int32_t)small(1);
  a.wrt = (int32_t)small(3);
  a.B = 1 + small(3);
  a.H = pick({1, 2, 4, 8});
  a.Hkv = chance(50) ? 0 : a.H / pick({1, 2, a.H});
  const int64_t hkv = a.Hkv > 0 ? a.Hkv : a.H;
  a.Sq = chance(10) ? 0 : pick({1, 7, 64, 100, 128, 300, 2048});
  a.Sk = chance(10) ? 0 : (chance(40) ? a.Sq : pick({1, 33, 64, 129, 1024}));
  a.D = pick({32, 64, 128});
  const void **ins[4] = {&a.q, &a.k, &a.v, &a.dy};
  void **outs[3] = {&a.dq, &a.dk, &a.dv};
  uintptr_t base = (uintptr_t)1 << 40;
  for (auto p : ins) *p = (const void *)(base += (uintptr_t)1 << 40);
  for (auto p : outs) *p = (void *)(base += (uintptr_t)1 << 40);
  const int64_t es = a.dtype == ATTN_BF16 ? 2 : 4;
  (void)es;
  int64_t *st[7] = {a.q_stride, a.k_stride, a.v_stride, a.dy_stride, a.dq_stride, a.dk_stride,
                    a.dv_stride};
  for (int i = 0; i < 7; ++i) {
    const bool qside = i == 0 || i == 3 || i == 4;
    contiguous(qside ? a.Sq : a.Sk, qside ? a.H : hkv, a.D, st[i]);
  }
  a.mask_kind = (int32_t)small(4);
  a.mask_flags = (a.mask_kind == 2 || a.mask_kind == 4) ? (int32_t)small(1) : 0;
  a.window = pick({0, 1, 256});
  a.mask = (const float *)(base += (uintptr_t)1 << 40);
  const int64_t ms[4] = {a.Sk, 0, 0, 1};
  std::memcpy(a.mask_stride, ms, sizeof ms);
  a.mask_threshold = 0.5f;
  a.scale = 0.0883883f;
  a.workspace = (void *)(base += (uintptr_t)1 << 40);
  a.workspace_bytes = attn_bwd_workspace_bytes(a.B, a.H, a.Sq);
  if (chance(30)) {
    switch (rng() % 8) {
      case 0: a.Sq = dim(); break;
      case 1: a.Sk = dim(); break;
      case 2: a.dk = (void *)a.k; break;
      case 3: st[rng() % 7][rng() % 3] = pick({-16, INT64_MAX, (int64_t)1 << 40, 8}); break;
      case 4: a.window = pick({-1, INT64_MAX, INT64_MIN}); break;
      case 5: a.workspace_bytes -= 1; break;
      case 6: a.mask_stride[rng() % 4] = pick({-1, INT64_MAX}); break;
      default: a.Hkv = pick({3, -2, a.H + 1}); break;
    }
  }
}

void fuzz_dense(long iters) {
  long ok = 0;
  for (long it = 0; it < iters; ++it) {
    attn_bwd_args a;
    std::memset(&a, 0, sizeof a);
    a.dtype = (int32_t)pick({0, 1, 1, 0, 2, -1});
    a.wrt = (int32_t)pick({3, 3, 3, 0, 1, 2, 4, -1});
    a.B = chance(85) ? pick({0, 1, 2, 4}) : dim();
    a.H = chance(85) ? pick({0, 1, 2, 4, 16}) : dim();
    a.Sq = dim();
    a.Sk = chance(30) ? a.Sq : dim();
    a.D = pick({32, 64, 128, 128, 0, 48, 256, -32});
    a.Hkv = chance(60) ? 0 : pick({1, 2, 3, -1, a.H, (int64_t)1 << 33});
    const int64_t hkv = a.Hkv > 0 ? a.Hkv : a.H;
    const void **ins[4] = {&a.q, &a.k, &a.v, &a.dy};
    void **outs[3] = {&a.dq, &a.dk, &a.dv};
    for (auto p : ins) *p = (const void *)fake_ptr();
    for (auto p : outs) *p = (void *)fake_ptr();
    if (chance(10)) a.dk = (void *)a.k;                  // aliasing
    if (chance(5) && a.dv) a.dq = (void *)((uintptr_t)a.dv + 64);  // overlap
    fill_strides(a.Sq, a.H, a.D, a.q_stride);
    fill_strides(a.Sk, hkv, a.D, a.k_stride);
    fill_strides(a.Sk, hkv, a.D, a.v_stride);
    fill_strides(a.Sq, a.H, a.D, a.dy_stride);
    fill_strides(a.Sq, a.H, a.D, a.dq_stride);
    fill_strides(a.Sk, hkv, a.D, a.dk_stride);
    fill_strides(a.Sk, hkv, a.D, a.dv_stride);
    a.mask_kind = (int32_t)pick({0, 1, 2, 3, 4, 1, 3, 5, -1});
    a.mask_flags = (int32_t)pick({0, 0, 1, 2});
    a.window = pick({0, 1, 256, 4096, -1, INT64_MAX, INT64_MIN, (int64_t)1 << 31});
    a.mask = (const float *)fake_ptr();
    for (int j = 0; j < 4; ++j) a.mask_stride[j] = pick({0, 1, 64, -1, INT64_MAX, a.Sk});
    a.mask_threshold = chance(5) ? std::nanf("") : 0.5f;
    static const float odd_scales[] = {0.f,       1e-30f,       -0.25f,          INFINITY,
                                       -INFINITY, std::nanf(""), 5.42101086e-20f, 3e38f};
    a.scale = chance(85) ? 0.125f : odd_scales[rng() % 8];
    const size_t need = chance(50) ? attn_bwd_workspace_bytes(a.B, a.H, a.Sq)
                                   : attn_bwd_split_workspace_bytes(a.B, a.H, a.Sq, a.Sk, a.D);
    a.workspace = (void *)fake_ptr();
    a.workspace_bytes = chance(80) ? need : (size_t)pick({0, 1, (int64_t)need - 1, INT64_MAX});

    if (chance(60)) make_valid(a);  // a well-formed call, perhaps with one field mutated
    int rc = attn_bwd(&a, nullptr);
    check_status(rc, "attn_bwd");
    ok += rc == ATTN_OK;
    check_status(attn_bwd_row_stats(&a, nullptr), "attn_bwd_row_stats");
    check_status(attn_bwd_kv(&a, nullptr), "attn_bwd_kv");
    check_status(attn_bwd_dq(&a, nullptr), "attn_bwd_dq");
    check_status(attn_bwd_stats_dq(&a, nullptr), "attn_bwd_stats_dq");
    int64_t ost[3];
    fill_strides(a.Sq, a.H, a.D, ost);
    const float *lse = (const float *)fake_ptr();
    const void *o = (const void *)fake_ptr();
    check_status(attn_bwd_from_forward(&a, lse, o, chance(5) ? nullptr : ost, nullptr),
                 "attn_bwd_from_forward");
  }
  std::fflush(stdout);
  std::printf("dense: %ld calls, %ld accepted by attn_bwd\n", iters * 6, ok);
}

// ---------------------------------------------------------------------------
// Paged planner and entry points.

// The structural promises the kernels rely on: every table inside the plan,
// every slot inside the pool, every row inside [0, nq * heads).
void check_plan(const std::vector<int32_t> &w, int32_t nseq, int32_t nq, int32_t heads,
                int32_t kv_heads, int32_t page_size, int32_t pool_pages) {
  using namespace attn::plan;
  const int64_t n = (int64_t)w.size();
  auto in = [&](int64_t off, int64_t cnt) {
    if (off < HEADER_WORDS || cnt < 0 || off + cnt > n) die("plan table outside the plan");
  };
  const int64_t items = w[W_ITEMS], links = w[W_LINKS], qh = w[W_QH];
  const int64_t slots = (int64_t)pool_pages * page_size;
  if (w[W_MAGIC] != kMagic || w[W_WORDS] != n) die("plan header");
  in(w[W_OFF_ITEM_LINKS], items + 1);
  in(w[W_OFF_ITEM_SLOTS], items * kItemSlots);
  in(w[W_OFF_LINK_SEQ], links);
  in(w[W_OFF_LINK_INFO], links * LINK_INFO_WORDS);
  in(w[W_OFF_LINK_TOK], links * kItemSlots);
  in(w[W_OFF_SEQ_QH], nseq + 1);
  in(w[W_OFF_QH_RH], qh);
  in(w[W_OFF_QH_POS], qh);
  in(w[W_OFF_SEQ_MAXPOS], nseq);
  in(w[W_OFF_SEQ_MINPOS], nseq);
  in(w[W_OFF_LISTED], w[W_LISTED]);
  in(w[W_OFF_SEQ_TOK], nseq + 1);
  in(w[W_OFF_TOK_SLOT], w[W_TOKENS]);
  in(w[W_OFF_QBLK], 2 * (int64_t)w[W_QBLK]);
  in(w[W_OFF_QPIECE], 3 * (int64_t)w[W_QPIECES]);
  in(w[W_OFF_QBLK_PIECE], (int64_t)w[W_QBLK] + 1);
  in(w[W_OFF_QPIECE_ORDER], w[W_QPIECES]);
  const int32_t *il = &w[w[W_OFF_ITEM_LINKS]];
  for (int64_t i = 0; i < items; ++i)
    if (il[i] < 0 || il[i] > il[i + 1] || il[i + 1] > links) die("item -> link CSR");
  const int32_t *sl = &w[w[W_OFF_ITEM_SLOTS]];
  for (int64_t i = 0; i < items * kItemSlots; ++i)
    if (sl[i] < -1 || (sl[i] >= 0 && sl[i] / 2 >= slots)) die("item slot outside the pool");
  for (int64_t l = 0; l < links; ++l)
    if (w[w[W_OFF_LINK_SEQ] + l] < 0 || w[w[W_OFF_LINK_SEQ] + l] >= nseq) die("link sequence");
  const int32_t *sq = &w[w[W_OFF_SEQ_QH]];
  for (int32_t s = 0; s < nseq; ++s)
    if (sq[s] < 0 || sq[s] > sq[s + 1] || sq[s + 1] > qh) die("sequence -> row CSR");
  for (int64_t l = 0; l < links; ++l) {  // the record's copy of its sequence's facts
    const int32_t *li = &w[w[W_OFF_LINK_INFO] + l * LINK_INFO_WORDS];
    const int32_t s = w[w[W_OFF_LINK_SEQ] + l];
    if (li[LI_SEQ] != s || li[LI_QH0] != sq[s] || li[LI_NQH] != sq[s + 1] - sq[s] ||
        li[LI_MINPOS] != w[w[W_OFF_SEQ_MINPOS] + s] || li[LI_MAXPOS] != w[w[W_OFF_SEQ_MAXPOS] + s])
      die("link record");
  }
  for (int64_t r = 0; r < qh; ++r) {
    const int32_t rh = w[w[W_OFF_QH_RH] + r];
    if (rh < 0 || (int64_t)rh >= (int64_t)nq * heads) die("qh row outside [0, nq * heads)");
    if (rh % heads >= heads / kv_heads) die("qh row's head outside its group");
  }
  for (int64_t t = 0; t < w[W_TOKENS]; ++t) {
    const int32_t s = w[w[W_OFF_TOK_SLOT] + t];
    if (s < 0 || s >= slots) die("token slot outside the pool");
  }
  for (int64_t b = 0; b < w[W_QBLK]; ++b) {
    const int32_t s = w[w[W_OFF_QBLK] + 2 * b], r0 = w[w[W_OFF_QBLK] + 2 * b + 1];
    if (s < 0 || s >= nseq || r0 < 0 || r0 >= qh) die("query block");
  }
  for (int64_t p = 0; p < w[W_QPIECES]; ++p) {
    const int32_t *pc = &w[w[W_OFF_QPIECE] + 3 * p];
    if (pc[0] < 0 || pc[0] >= w[W_QBLK] || pc[1] < 0 || pc[1] > pc[2]) die("query piece");
    const int32_t o = w[w[W_OFF_QPIECE_ORDER] + p];
    if (o < 0 || o >= w[W_QPIECES]) die("query piece order");
  }
}

void call_paged(const std::vector<int32_t> &plan, int32_t nq, int32_t heads, int32_t kv_heads,
                int32_t page_size, int32_t pool_pages) {
  attn_bwd_paged_args a;
  std::memset(&a, 0, sizeof a);
  a.dtype = (int32_t)pick({0, 1, 1, 3});
  a.need = (int32_t)pick({1, 2, 3, 3, 0, 4, 5});
  a.heads = chance(90) ? heads : heads + 1;
  a.kv_heads = kv_heads;
  a.head_dim = (int32_t)pick({32, 64, 128, 128, 96, 192, 256});
  a.page_size = page_size;
  a.causal = (int32_t)pick({0, 1, 1, 2});
  a.kv_workgroups = (int32_t)(chance(90) ? pick({0, 0, 8, 256, -1}) : pick({-2, INT32_MIN}));
  a.nq = chance(95) ? nq : nq + 1;
  a.pool_pages = pool_pages;
  a.scale = chance(90) ? 0.088f : std::nanf("");
  a.q = (const void *)fake_ptr();
  a.dy = (const void *)fake_ptr();
  a.k_pool = (const void *)fake_ptr();
  a.v_pool = (const void *)fake_ptr();
  a.stats = (const float *)fake_ptr();
  a.plan_host = plan.data();
  a.plan = (const int32_t *)fake_ptr();
  a.dk_pool = (void *)fake_ptr();
  a.dv_pool = (void *)fake_ptr();
  if (chance(20)) {
    a.mla = (int32_t)pick({1, 1, 2});
    a.position_dim = (int32_t)pick({0, 32, 64, 16});
    a.qp = (const void *)fake_ptr();
    a.kp_pool = (const void *)fake_ptr();
    a.dkp_pool = (void *)fake_ptr();
  }
  check_status(attn_bwd_paged(&a, nullptr), "attn_bwd_paged");
  const size_t qws = attn_bwd_paged_q_workspace_bytes(plan.data(), a.head_dim);
  if (chance(50)) {
    a.q_workspace = (void *)fake_ptr();
    a.q_workspace_bytes = chance(80) ? qws : qws / 2;
  }
  a.mla = chance(10) ? 1 : 0;
  check_status(attn_bwd_paged_row_stats(&a, (float *)fake_ptr(), nullptr), "paged_row_stats");
  check_status(attn_bwd_paged_dq(&a, (void *)fake_ptr(), nullptr), "paged_dq");
  a.q_form = (int32_t)pick({0, 1, 2, 3, -1});
  check_status(attn_bwd_paged_stats_dq(&a, (float *)fake_ptr(), (void *)fake_ptr(), nullptr),
               "paged_stats_dq");
}

void fuzz_paged(long iters) {
  long built = 0, words_rej = 0, build_rej = 0;
  for (long it = 0; it < iters; ++it) {
    const int32_t nseq = (int32_t)small(5);
    const int32_t page_size = (int32_t)(chance(96) ? pick({1, 4, 16, 16, 48, 256}) : pick({0, -1}));
    std::vector<int32_t> lens(nseq);
    for (auto &l : lens)
      l = (int32_t)(chance(98) ? small(300) : pick({-1, 1 << 30, INT32_MAX}));
    int64_t needp = 0;
    for (int32_t l : lens)
      if (page_size > 0 && l > 0) needp = std::max<int64_t>(needp, ((int64_t)l + page_size - 1) / page_size);
    const int32_t max_pages = (int32_t)(chance(96) ? needp + small(2) : pick({0, needp - 1}));
    int64_t total = 0;
    for (int32_t l : lens)
      if (page_size > 0 && l > 0) total += ((int64_t)l + page_size - 1) / page_size;
    const int32_t pool_pages =
        (int32_t)(chance(96) ? std::min<int64_t>(total + small(8), 1 << 20) : pick({0, 1 << 29, -3}));
    const int32_t kv_heads = (int32_t)(chance(95) ? pick({1, 2, 4, 8}) : 0);
    const int32_t heads = (int32_t)(kv_heads * pick({1, 2, 4}) + (chance(5) ? 1 : 0));
    const int32_t nq = (int32_t)(chance(95) ? small(20) : pick({-1, 1 << 28}));
    std::vector<int32_t> qs(std::max(nq, 0) < 64 ? std::max(nq, 0) : 64), qp(qs.size());
    for (size_t r = 0; r < qs.size(); ++r) {
      qs[r] = nseq > 0 ? (int32_t)(rng() % (uint64_t)nseq) : 0;
      qp[r] = (int32_t)small(320);
      if (chance(1)) qs[r] = (int32_t)pick({-1, nseq});
      if (chance(1)) qp[r] = (int32_t)pick({-1, INT32_MAX});
    }
    const int32_t nq_used = (int32_t)qs.size() == nq ? nq : (nq < 0 ? nq : (int32_t)qs.size());
    const int64_t words = attn_bwd_paged_plan_words(nseq, lens.data(), max_pages, nq_used, heads,
                                                    kv_heads, page_size, pool_pages);
    if (words < 0) {
      ++words_rej;
      if (attn_bwd_last_error()[0] == '\0') die("plan_words rejection without a message");
      continue;
    }
    if (words > (1 << 20) || (int64_t)nseq * max_pages > (1 << 20))
      continue;  // a legal but very large plan: not built here
    std::vector<int32_t> bt((size_t)std::max<int64_t>(0, (int64_t)nseq * std::max(max_pages, 0)));
    for (auto &e : bt) {
      e = pool_pages > 0 ? (int32_t)(rng() % (uint64_t)pool_pages) : 0;
      if (chance(1)) e = (int32_t)pick({-1, pool_pages, INT32_MAX});
    }
    if (nseq >= 2 && max_pages > 0 && chance(30)) bt[max_pages] = bt[0];  // a shared first page
    std::vector<int32_t> buf((size_t)words);
    const int rc = attn_bwd_paged_plan_build(nseq, lens.data(), bt.data(), max_pages, nq_used,
                                             qs.data(), qp.data(), heads, kv_heads, page_size,
                                             pool_pages, buf.data(), words);
    check_status(rc, "attn_bwd_paged_plan_build");
    if (rc != ATTN_OK) {
      ++build_rej;
      if (std::getenv("ABI_FUZZ_VERBOSE")) std::fprintf(stderr, "build: %s\n", attn_bwd_last_error());
      continue;
    }
    ++built;
    // An exact-size copy, so that any read past the plan is an ASan error.
    std::vector<int32_t> plan(buf.begin(), buf.begin() + buf[attn::plan::W_WORDS]);
    check_plan(plan, nseq, nq_used, heads, kv_heads, page_size, pool_pages);
    call_paged(plan, nq_used, heads, kv_heads, page_size, pool_pages);
    // A corrupted offset or count in the header must be refused or stay in the header.
    std::vector<int32_t> bad = plan;
    const int wsel = (int)(attn::plan::W_NSEQ + rng() % (attn::plan::HEADER_WORDS - attn::plan::W_NSEQ));
    bad[wsel] = (int32_t)pick({-1, 0, INT32_MAX, (int64_t)plan.size() + 5, 1 << 20});
    call_paged(bad, nq_used, heads, kv_heads, page_size, pool_pages);
  }
  std::printf("paged: %ld plans built, %ld refused by plan_words, %ld by plan_build\n", built,
              words_rej, build_rej);
}

}  // namespace

int main(int argc, char **argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 2000;
  rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
  fuzz_dense(iters);
  fuzz_paged(iters);
  std::printf("launch stubs reached: %ld\n", n_launch);
  return 0;
}
