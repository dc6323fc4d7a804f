"""Host-side checks of the C ABI (no GPU needed, no compute call is made):
the library loads, exports every function include/attn_bwd.h declares, and its
validation rejects bad arguments before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import scaled_dot_product_bwd_amd as sdb
from scaled_dot_product_bwd_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(attn_bwd\w*)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = sdb.load_library()
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert declared == set(_abi.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_bwd\w*)", out))
    assert declared <= exported, declared - exported
    for name in declared:
        assert getattr(lib, name) is not None


def test_args_struct_size_matches_header_layout():
    # 2 int32 + 5 int64 + 7 pointers + 21 int64 strides + 2 int32 + int64 window
    # + pointer + 4 int64 + 2 float + pointer + size_t + int64 Hkv
    assert ctypes.sizeof(_abi.AttnBwdArgs) == 8 + 40 + 56 + 168 + 8 + 8 + 8 + 32 + 8 + 8 + 8 + 8


def test_workspace_bytes():
    assert sdb.workspace_bytes(4, 16, 2048) == 4 * 4 * 16 * 2048 * 4
    assert sdb.workspace_bytes(1, 1, 1) == 4 * 256
    assert sdb.workspace_bytes(0, 3, 5) == 0


def _args(**kw):
    a = _abi.AttnBwdArgs()
    a.dtype, a.wrt, a.B, a.H, a.Sq, a.Sk, a.D = 1, 3, 1, 2, 64, 64, 64
    base = 1 << 20  # fake, 256-aligned addresses: only validated, never touched
    for i, name in enumerate(("q", "k", "v", "dy", "dq", "dk", "dv")):
        setattr(a, name, base * (i + 1))
        getattr(a, name + "_stride")[:] = (64 * 2 * 64, 2 * 64, 64)
    a.scale = 0.125
    a.workspace = base * 16
    a.workspace_bytes = sdb.workspace_bytes(1, 2, 64)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def _rc(a):
    lib = sdb.load_library()
    rc = lib.attn_bwd(ctypes.byref(a), None)
    return rc, lib.attn_bwd_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 5, _abi.ATTN_E_INVALID),
    ("wrt", 4, _abi.ATTN_E_INVALID),
    ("mask_kind", 9, _abi.ATTN_E_INVALID),
    ("D", 96, _abi.ATTN_E_UNSUPPORTED),
    ("Hkv", 3, _abi.ATTN_E_INVALID),   # H = 2 is not a multiple of 3
    ("Hkv", -1, _abi.ATTN_E_INVALID),
    ("D", 256, _abi.ATTN_E_UNSUPPORTED),
    ("Sq", -1, _abi.ATTN_E_INVALID),
    ("q", 0, _abi.ATTN_E_INVALID),
    ("dk", 0, _abi.ATTN_E_INVALID),
    ("q", (1 << 20) + 8, _abi.ATTN_E_UNSUPPORTED),
    ("workspace", 0, _abi.ATTN_E_WORKSPACE),
    ("workspace_bytes", 100, _abi.ATTN_E_WORKSPACE),
    ("scale", float("inf"), _abi.ATTN_E_INVALID),
    ("scale", 0.0, _abi.ATTN_E_UNSUPPORTED),
    ("scale", -1e-30, _abi.ATTN_E_UNSUPPORTED),
    ("scale", 3e38, _abi.ATTN_E_UNSUPPORTED),  # scale * log2(e) would overflow to inf
    ("mask_flags", 1, _abi.ATTN_E_INVALID),   # the causal flag needs KEYPAD or BIAS
])
def test_validation_rejects(field, value, code):
    rc, msg = _rc(_args(**{field: value}))
    assert rc == code, (rc, msg)
    assert msg


def test_validation_rejects_window_and_mask_problems():
    rc, _ = _rc(_args(mask_kind=_abi.ATTN_MASK_WINDOW, window=-3))
    assert rc == _abi.ATTN_E_INVALID
    rc, msg = _rc(_args(mask_kind=_abi.ATTN_MASK_BIAS))
    assert rc == _abi.ATTN_E_INVALID and "mask" in msg
    a = _args()
    a.q_stride[1] = 4  # 8-byte row stride for bf16: rows not 16-byte aligned
    assert _rc(a)[0] == _abi.ATTN_E_UNSUPPORTED


def test_validation_rejects_aliasing():
    a = _args()
    a.dk = a.k
    rc, msg = _rc(a)
    assert rc == _abi.ATTN_E_INVALID and "overlaps" in msg
    a = _args()
    a.dv = a.dq
    assert _rc(a)[0] == _abi.ATTN_E_INVALID
    a = _args()
    a.dq = a.workspace
    assert _rc(a)[0] == _abi.ATTN_E_INVALID


@pytest.mark.parametrize("entry", ["attn_bwd_row_stats", "attn_bwd_kv", "attn_bwd_dq",
                                   "attn_bwd_stats_dq"])
def test_stage_entries_validate_like_attn_bwd(entry):
    """The stage entry points take attn_bwd's validation before any launch."""
    lib = sdb.load_library()
    for field, value, code in (("D", 96, _abi.ATTN_E_UNSUPPORTED), ("q", 0, _abi.ATTN_E_INVALID),
                               ("workspace", 0, _abi.ATTN_E_WORKSPACE)):
        a = _args(**{field: value})
        assert getattr(lib, entry)(ctypes.byref(a), None) == code, (entry, field)
    a = _args()
    a.dq = a.k  # output over an input
    assert getattr(lib, entry)(ctypes.byref(a), None) == _abi.ATTN_E_INVALID


def test_unrequested_outputs_may_be_null():
    # wrt = Q with dk = dv = NULL passes validation up to the first check that
    # needs a real device; give it a NULL q to stop there instead.
    a = _args(wrt=_abi.ATTN_WRT_Q, dk=0, dv=0, q=0)
    rc, msg = _rc(a)
    assert rc == _abi.ATTN_E_INVALID and msg.startswith("q is NULL")


# ---------------------------------------------------------------------------
# attn_bwd_paged: validation happens on the host before any launch.

def test_paged_args_struct_size():
    # 9 int32 + float, then 9 pointers, the latent variant's 2 int32 + 3 pointers,
    # the query side's workspace pointer and size, kv_workgroups (+ tail padding)
    assert ctypes.sizeof(_abi.AttnBwdPagedArgs) == 40 + 9 * 8 + 8 + 3 * 8 + 16 + 8


def _paged_plan(heads=4, kv_heads=2):
    import numpy as np
    lens = np.array([20, 9], np.int32)
    bt = np.array([[3, 0], [1, -1]], np.int32)
    qs = np.array([0, 0, 1], np.int32)
    qp = np.array([18, 19, 8], np.int32)
    return sdb.paged_plan(lens, bt, qs, qp, heads=heads, kv_heads=kv_heads, page_size=16,
                          pool_pages=4)


def _paged_args(the_plan, **kw):
    a = _abi.AttnBwdPagedArgs()
    a.dtype, a.need, a.heads, a.kv_heads, a.head_dim = 1, 3, 4, 2, 64
    a.page_size, a.causal, a.nq, a.pool_pages, a.scale = 16, 1, 3, 4, 0.125
    base = 1 << 24  # fake, aligned, disjoint addresses: only validated, never touched
    for i, name in enumerate(("q", "dy", "k_pool", "v_pool", "stats", "plan", "dk_pool",
                              "dv_pool")):
        setattr(a, name, base * (i + 1))
    a.plan_host = the_plan.words.ctypes.data
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def _paged_rc(a):
    lib = sdb.load_library()
    rc = lib.attn_bwd_paged(ctypes.byref(a), None)
    return rc, lib.attn_bwd_last_error().decode()


@pytest.mark.parametrize("field,value,code,msg", [
    ("dtype", 2, _abi.ATTN_E_INVALID, "dtype"),
    ("need", 0, _abi.ATTN_E_INVALID, "need"),
    ("need", 4, _abi.ATTN_E_INVALID, "need"),
    ("head_dim", 48, _abi.ATTN_E_UNSUPPORTED, "head_dim"),
    ("causal", 2, _abi.ATTN_E_INVALID, "causal"),
    ("heads", 8, _abi.ATTN_E_INVALID, "plan was built"),
    ("page_size", 8, _abi.ATTN_E_INVALID, "plan was built"),
    ("nq", 4, _abi.ATTN_E_INVALID, "plan was built"),
    ("pool_pages", 5, _abi.ATTN_E_INVALID, "plan was built"),
    ("plan", 0, _abi.ATTN_E_INVALID, "plan"),
    ("kv_workgroups", -2, _abi.ATTN_E_INVALID, "kv_workgroups"),
    ("q", 0, _abi.ATTN_E_INVALID, "q is NULL"),
    ("stats", (1 << 24) * 5 + 4, _abi.ATTN_E_UNSUPPORTED, "aligned"),
    ("dk_pool", 0, _abi.ATTN_E_INVALID, "dk_pool is NULL"),
    ("dv_pool", (1 << 24) * 3, _abi.ATTN_E_INVALID, "overlaps"),
    ("scale", float("inf"), _abi.ATTN_E_INVALID, "scale"),
    ("scale", 0.0, _abi.ATTN_E_UNSUPPORTED, "scale"),
])
def test_paged_rejections(field, value, code, msg):
    plan = _paged_plan()
    rc, err = _paged_rc(_paged_args(plan, **{field: value}))
    assert rc == code and msg in err, (rc, err)


_MLA = dict(mla=1, need=5, position_dim=32, v_pool=0, dv_pool=0, qp=(1 << 24) * 9,
            kp_pool=(1 << 24) * 10, dkp_pool=(1 << 24) * 11)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(mla=2), _abi.ATTN_E_INVALID, "mla"),
    (dict(_MLA, need=2), _abi.ATTN_E_INVALID, "need"),
    (dict(_MLA, need=3), _abi.ATTN_E_INVALID, "need"),
    (dict(_MLA, need=8), _abi.ATTN_E_INVALID, "need"),
    (dict(_MLA, head_dim=32), _abi.ATTN_E_UNSUPPORTED, "latent width"),
    (dict(_MLA, head_dim=320), _abi.ATTN_E_UNSUPPORTED, "latent width"),
    (dict(_MLA, head_dim=192, dtype=0), _abi.ATTN_E_UNSUPPORTED, "latent width"),  # fp32: 64 / 128
    (dict(_MLA, head_dim=256, dtype=0), _abi.ATTN_E_UNSUPPORTED, "latent width"),
    (dict(_MLA, position_dim=16), _abi.ATTN_E_UNSUPPORTED, "position_dim"),
    (dict(_MLA, position_dim=0), _abi.ATTN_E_INVALID, "position_dim is 0"),
    (dict(_MLA, qp=0), _abi.ATTN_E_INVALID, "qp is NULL"),
    (dict(_MLA, kp_pool=0), _abi.ATTN_E_INVALID, "kp_pool is NULL"),
    (dict(_MLA, dkp_pool=0), _abi.ATTN_E_INVALID, "dkp_pool is NULL"),
    (dict(_MLA, dkp_pool=(1 << 24) * 10), _abi.ATTN_E_INVALID, "overlaps"),
    (dict(_MLA, dk_pool=(1 << 24) * 9), _abi.ATTN_E_INVALID, "overlaps"),
    (dict(_MLA, dkp_pool=(1 << 24) * 6), _abi.ATTN_E_INVALID, "overlaps"),  # the plan
    (dict(_MLA, kp_pool=(1 << 24) * 10 + 8), _abi.ATTN_E_UNSUPPORTED, "aligned"),
])
def test_paged_latent_rejections(kw, code, msg):
    plan = _paged_plan()
    rc, err = _paged_rc(_paged_args(plan, **kw))
    assert rc == code and msg in err, (rc, err)


def test_paged_query_workspace_rules():
    plan = _paged_plan()
    lib = sdb.load_library()
    W = plan.words
    need_dq = int(W[_abi.W_QPIECES]) * 2 * 128 * 64 * 4  # pieces * kv_heads * rows * D * 4
    need_all = int(W[_abi.W_QPIECES]) * 2 * 128 * (2 * 64 + 8) * 4  # the fused call's records
    assert lib.attn_bwd_paged_q_workspace_bytes(W.ctypes.data, 64) == need_all
    bad = W.copy()
    bad[0] = 7
    assert lib.attn_bwd_paged_q_workspace_bytes(bad.ctypes.data, 64) == 0
    out = ctypes.c_void_p(1 << 30)
    a = _paged_args(plan, q_workspace=(1 << 24) * 12, q_workspace_bytes=need_dq - 4)
    assert lib.attn_bwd_paged_dq(ctypes.byref(a), out, None) == _abi.ATTN_E_WORKSPACE
    a = _paged_args(plan, q_workspace=(1 << 24) * 12 + 8, q_workspace_bytes=need_dq)
    assert lib.attn_bwd_paged_dq(ctypes.byref(a), out, None) == _abi.ATTN_E_UNSUPPORTED
    a = _paged_args(plan, q_workspace=(1 << 24) * 1, q_workspace_bytes=need_dq)  # over q
    assert lib.attn_bwd_paged_dq(ctypes.byref(a), out, None) == _abi.ATTN_E_INVALID
    assert "q_workspace overlaps" in lib.attn_bwd_last_error().decode()
    # the fused call (bf16) keeps 2 D + 8 floats per row and piece
    st = ctypes.c_void_p((1 << 24) * 13)
    a = _paged_args(plan, q_workspace=(1 << 24) * 12, q_workspace_bytes=need_all - 4)
    assert lib.attn_bwd_paged_stats_dq(ctypes.byref(a), st, out, None) == _abi.ATTN_E_WORKSPACE
    assert str(need_all) in lib.attn_bwd_last_error().decode()
    a = _paged_args(plan, q_workspace=(1 << 24) * 13, q_workspace_bytes=need_all)  # over stats
    assert lib.attn_bwd_paged_stats_dq(ctypes.byref(a), st, out, None) == _abi.ATTN_E_INVALID
    assert "q_workspace overlaps" in lib.attn_bwd_last_error().decode()


def test_paged_query_side_rejects_latent_variant():
    plan = _paged_plan()
    lib = sdb.load_library()
    a = _paged_args(plan, **_MLA)
    for fn in (lib.attn_bwd_paged_row_stats, lib.attn_bwd_paged_dq):
        assert fn(ctypes.byref(a), ctypes.c_void_p(1 << 30), None) == _abi.ATTN_E_UNSUPPORTED
        assert "latent" in lib.attn_bwd_last_error().decode()
    assert lib.attn_bwd_paged_stats_dq(ctypes.byref(a), ctypes.c_void_p(1 << 30),
                                       ctypes.c_void_p(3 << 29), None) == _abi.ATTN_E_UNSUPPORTED


def test_paged_rejects_foreign_plan():
    import numpy as np
    plan = _paged_plan()
    words = plan.words.copy()
    words[0] = 12345
    a = _paged_args(plan)
    a.plan_host = words.ctypes.data
    rc, err = _paged_rc(a)
    assert rc == _abi.ATTN_E_INVALID and "magic" in err
    words = plan.words.copy()
    words[_abi.W_OFF_LINK_TOK] = 10 ** 8
    a.plan_host = words.ctypes.data
    rc, err = _paged_rc(a)
    assert rc == _abi.ATTN_E_INVALID and "offsets" in err
    assert np.array_equal(plan.words[:2], [_abi.PLAN_MAGIC, len(plan.words)])


def test_paged_empty_plan_is_a_no_op():
    import numpy as np
    plan = sdb.paged_plan(np.zeros(1, np.int32), np.zeros((1, 1), np.int32), np.zeros(0, np.int32),
                          np.zeros(0, np.int32), heads=4, kv_heads=2, page_size=16, pool_pages=4)
    assert plan.items == 0
    a = _paged_args(plan, nq=0)
    for name in ("q", "dy", "k_pool", "v_pool", "stats", "dk_pool", "dv_pool"):
        setattr(a, name, 0)
    assert _paged_rc(a)[0] == _abi.ATTN_OK


def test_paged_query_side_rejections():
    plan = _paged_plan()
    lib = sdb.load_library()
    a = _paged_args(plan)
    for fn in (lib.attn_bwd_paged_row_stats, lib.attn_bwd_paged_dq):
        assert fn(ctypes.byref(a), None, None) == _abi.ATTN_E_INVALID      # no output
        assert "NULL" in lib.attn_bwd_last_error().decode()
        assert fn(ctypes.byref(a), ctypes.c_void_p(a.q), None) == _abi.ATTN_E_INVALID  # aliases q
        assert "overlaps" in lib.attn_bwd_last_error().decode()
    a.stats = 0   # the statistics kernel does not read the input statistics
    a.need = 0    # nor `need`
    assert lib.attn_bwd_paged_row_stats(ctypes.byref(a), None, None) == _abi.ATTN_E_INVALID
    assert "stats_out is NULL" in lib.attn_bwd_last_error().decode()
    assert lib.attn_bwd_paged_dq(ctypes.byref(a), ctypes.c_void_p(1 << 30), None) == _abi.ATTN_E_INVALID
    assert "stats is NULL" in lib.attn_bwd_last_error().decode()
    # the fused call: two outputs, neither NULL, disjoint from each other and the inputs
    fused = lib.attn_bwd_paged_stats_dq
    st, dq = ctypes.c_void_p(1 << 30), ctypes.c_void_p(3 << 29)
    assert fused(ctypes.byref(a), None, dq, None) == _abi.ATTN_E_INVALID
    assert "stats_out is NULL" in lib.attn_bwd_last_error().decode()
    assert fused(ctypes.byref(a), st, None, None) == _abi.ATTN_E_INVALID
    assert "dq is NULL" in lib.attn_bwd_last_error().decode()
    assert fused(ctypes.byref(a), st, st, None) == _abi.ATTN_E_INVALID
    assert "overlaps" in lib.attn_bwd_last_error().decode()
    assert fused(ctypes.byref(a), st, ctypes.c_void_p(a.dy), None) == _abi.ATTN_E_INVALID
    assert "overlaps" in lib.attn_bwd_last_error().decode()
    for bad in (3, -1):
        a.q_form = bad
        assert fused(ctypes.byref(a), st, dq, None) == _abi.ATTN_E_INVALID
        assert "q_form" in lib.attn_bwd_last_error().decode()
    a.q_form = 1  # the split form without a workspace
    assert fused(ctypes.byref(a), st, dq, None) == _abi.ATTN_E_WORKSPACE
    assert "q_workspace" in lib.attn_bwd_last_error().decode()


def test_from_forward_rejections():
    lib = sdb.load_library()
    a = _args()
    ost = (ctypes.c_int64 * 3)(64 * 2 * 64, 2 * 64, 64)
    rc = lib.attn_bwd_from_forward(ctypes.byref(a), None, ctypes.c_void_p(1 << 28), ost, None)
    assert rc == _abi.ATTN_E_INVALID and "NULL" in lib.attn_bwd_last_error().decode()
    rc = lib.attn_bwd_from_forward(ctypes.byref(a), ctypes.c_void_p(1 << 29), ctypes.c_void_p((1 << 28) + 2),
                                   ost, None)
    assert rc == _abi.ATTN_E_UNSUPPORTED and "aligned" in lib.attn_bwd_last_error().decode()
    # lse inside the workspace
    rc = lib.attn_bwd_from_forward(ctypes.byref(a), ctypes.c_void_p(a.workspace), ctypes.c_void_p(1 << 28),
                                   ost, None)
    assert rc == _abi.ATTN_E_INVALID and "workspace" in lib.attn_bwd_last_error().decode()


def test_validation_survives_huge_strides_and_sizes():
    """Byte extents are computed exactly: a stride or size whose extent passes
    2^60 bytes is refused instead of wrapping into a wrong overlap decision."""
    for field, j, value in (("k_stride", 0, 2 ** 63 - 1), ("dq_stride", 1, 2 ** 61),
                            ("q_stride", 2, 2 ** 62)):
        a = _args()
        getattr(a, field)[j] = value
        rc, msg = _rc(a)
        assert rc in (_abi.ATTN_E_INVALID, _abi.ATTN_E_UNSUPPORTED), (field, rc, msg)
    rc, msg = _rc(_args(B=2 ** 40, H=2 ** 40))
    assert rc == _abi.ATTN_E_INVALID and "too large" in msg
    assert sdb.workspace_bytes(2 ** 40, 2 ** 20, 2 ** 20) == 2 ** 64 - 1  # never satisfiable
