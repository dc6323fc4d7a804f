"""Pins of the CPU float64 oracle to facts that do not come from the oracle.

Every pin compares the oracle with something independent of it: a worked
example computed by hand, hand-derived mask patterns, closed forms, invariants
of the exact mathematics, central finite differences of a forward pass computed
by torch's own scaled_dot_product_attention, and torch float64 autograd through
that same library routine.  None of these needs a GPU.

Mask rules: rlx-cpu 0.2.17 src/attention_bwd.rs (`apply_synthetic_mask`,
`backward_dense_head_all`); rlx-wgpu 0.2.1 attention_bwd.wgsl (`mask_score`).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import MASK_BIAS, MASK_CAUSAL, MASK_KEYPAD, MASK_NONE, MASK_WINDOW

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _to_bhsd(x):
    return torch.from_numpy(np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3))))


def _from_bhsd(t):
    return np.transpose(t.detach().numpy(), (0, 2, 1, 3))


def visible_from_rules(kind, Sq, Sk, window=0, valid=None, threshold=0.5, causal_flag=False):
    """Boolean [Sq, Sk] visibility per the page rules.  This helper is itself
    pinned against the hand-derived patterns in golden/visibility.json below."""
    off = max(Sk - Sq, 0)
    vis = np.ones((Sq, Sk), dtype=bool)
    i = np.arange(Sq)[:, None] + off
    j = np.arange(Sk)[None, :]
    if kind == MASK_KEYPAD:
        vis &= (np.asarray(valid)[None, :] >= threshold)
    if kind == MASK_CAUSAL or (kind in (MASK_KEYPAD, MASK_BIAS) and causal_flag):
        vis &= j <= i
    if kind == MASK_WINDOW:
        vis &= (j >= np.maximum(i - window, 0)) & (j <= i)
    return vis


def torch_reference(q, k, v, dy, vis=None, bias=None, scale=None):
    """float64 CPU autograd through torch.nn.functional.scaled_dot_product_attention.
    vis: bool [B or 1, H or 1, Sq, Sk]; bias: additive float [.., Sq, Sk]."""
    D = q.shape[-1]
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    qt, kt, vt = (_to_bhsd(x).requires_grad_(True) for x in (q, k, v))
    mask = None
    if vis is not None and bias is not None:
        mask = torch.from_numpy(np.where(vis, bias, -np.inf))
    elif vis is not None:
        mask = torch.from_numpy(np.asarray(vis))
    elif bias is not None:
        mask = torch.from_numpy(np.asarray(bias, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    (o * _to_bhsd(dy)).sum().backward()
    return dict(dq=_from_bhsd(qt.grad), dk=_from_bhsd(kt.grad), dv=_from_bhsd(vt.grad),
                out=_from_bhsd(o))


def rel_err(a, b):
    """max|a - b| / max|b|, with the denominator floored at 1 (inputs are O(1),
    so an exactly-zero reference is compared in absolute terms)."""
    den = max(np.max(np.abs(b)), 1.0)
    return np.max(np.abs(a - b)) / den


# ---------------------------------------------------------------- worked example
def test_worked_example_by_hand():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    i, e = ex["inputs"], ex["expected"]
    q = np.array(i["q"]).reshape(1, 1, 1, 1)
    k = np.array(i["k"]).reshape(1, 2, 1, 1)
    v = np.array(i["v"]).reshape(1, 2, 1, 1)
    dy = np.array(i["dy"]).reshape(1, 1, 1, 1)
    r = oracle.attn_bwd(q, k, v, dy, scale=i["scale"])
    np.testing.assert_allclose(r["dq"].ravel(), e["dq"], rtol=1e-13)
    np.testing.assert_allclose(r["dk"].ravel(), e["dk"], rtol=1e-13)
    np.testing.assert_allclose(r["dv"].ravel(), e["dv"], rtol=1e-13)
    np.testing.assert_allclose(r["m"].ravel(), [e["m"]], rtol=1e-13)
    np.testing.assert_allclose(r["l"].ravel(), [e["l"]], rtol=1e-13)
    np.testing.assert_allclose(r["delta"].ravel(), [e["delta"]], rtol=1e-13)
    np.testing.assert_allclose(r["out"].ravel(), [e["out"]], rtol=1e-13)


# ---------------------------------------------------------------- mask patterns
def _visibility_cases():
    return json.load(open(os.path.join(GOLDEN, "visibility.json")))["cases"]


@pytest.mark.parametrize("case", _visibility_cases(), ids=lambda c: c["name"])
def test_visibility_matches_hand_patterns(case):
    """With Q = 0 every visible score is 0, so P is uniform over the visible set
    V_i; with dY_i = e_i (one-hot), dV_j[i] = [j in V_i] / |V_i| reveals V_i."""
    Sq, Sk = case["Sq"], case["Sk"]
    D = max(Sq, 1)
    q = np.zeros((1, Sq, 1, D))
    k = _rand((1, Sk, 1, D), 1)
    v = _rand((1, Sk, 1, D), 2)
    dy = np.eye(Sq, D).reshape(1, Sq, 1, D)
    valid = np.array(case.get("valid", [1.0] * Sk))
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=case["kind"], window=case["window"],
                        mask=valid.reshape(1, 1, 1, Sk), threshold=case.get("threshold", 0.5),
                        causal_flag=case.get("causal_flag", 0))
    want = np.array([[c == "1" for c in row] for row in case["pattern"]])
    got = r["dv"][0, :, 0, :Sq].T  # [Sq, Sk]: got[i, j] = dV_j[i]
    assert np.array_equal(got > 0, want), (got, want)
    for i in range(Sq):
        n = want[i].sum()
        if n:
            np.testing.assert_allclose(got[i][want[i]], 1.0 / n, rtol=1e-14)
        else:  # fully masked row: no contribution anywhere, zero statistics
            assert r["l"][0, 0, i] == 0.0 and r["delta"][0, 0, i] == 0.0
            assert r["m"][0, 0, i] == -np.inf
            assert np.all(r["dq"][0, i] == 0.0)
    # the helper used by the torch comparisons below agrees with the hand patterns
    assert np.array_equal(visible_from_rules(case["kind"], Sq, Sk, case["window"], valid,
                                             case.get("threshold", 0.5),
                                             case.get("causal_flag", 0)), want)


# ---------------------------------------------------------------- library routine
SHAPES = [(1, 1, 1, 1, 4), (2, 2, 5, 5, 4), (1, 2, 3, 8, 8), (2, 1, 8, 3, 4), (1, 2, 17, 33, 16)]


@pytest.mark.parametrize("B,H,Sq,Sk,D", SHAPES)
@pytest.mark.parametrize("kind", ["none", "causal", "window", "keypad", "bias", "keypad_causal",
                                  "bias_causal"])
def test_against_torch_sdpa_autograd(B, H, Sq, Sk, D, kind):
    q, k, v, dy = (_rand(s, n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                        (B, Sk, H, D), (B, Sq, H, D)]))
    g = np.random.default_rng(99)
    mask_kind, window, mask, causal_flag, bias = MASK_NONE, 0, None, False, None
    vis = np.ones((B, 1, Sq, Sk), dtype=bool)
    if kind == "causal":
        mask_kind = MASK_CAUSAL
        vis[:] = visible_from_rules(MASK_CAUSAL, Sq, Sk)
    elif kind == "window":
        mask_kind, window = MASK_WINDOW, 2
        vis[:] = visible_from_rules(MASK_WINDOW, Sq, Sk, 2)
    elif kind.startswith("keypad"):
        mask_kind, causal_flag = MASK_KEYPAD, kind.endswith("causal")
        valid = (g.random((B, Sk)) > 0.3).astype(np.float64)
        valid[:, 0] = 1.0  # keep every row non-empty: torch gives NaN for empty rows
        mask = valid.reshape(B, 1, 1, Sk)
        for b in range(B):
            vis[b, 0] = visible_from_rules(MASK_KEYPAD, Sq, Sk, 0, valid[b], 0.5, causal_flag)
    elif kind.startswith("bias"):
        mask_kind, causal_flag = MASK_BIAS, kind.endswith("causal")
        bias = g.standard_normal((B, H, Sq, Sk))
        mask = bias
        vis[:] = visible_from_rules(MASK_BIAS, Sq, Sk, causal_flag=causal_flag)
    if not vis.any(axis=-1).all():
        pytest.skip("a fully masked row: torch returns NaN there (pinned separately)")
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=mask_kind, window=window, mask=mask,
                        causal_flag=causal_flag, nthreads=2)
    ref = torch_reference(q, k, v, dy, vis=vis, bias=bias)
    for name in ("dq", "dk", "dv", "out"):
        assert rel_err(r[name], ref[name]) < 1e-12, name


def test_p1_unit_test_shape_against_torch():
    """The shape and generator of the rlx-cpu unit test `all_matches_three_separate`
    (b2 h2 s5 d4, causal, [B, S, H, D])."""
    import sdpa_inputs
    n = 2 * 5 * 2 * 4
    q, k, v, dy = (sdpa_inputs.hash_inputs(n, s).double().numpy().reshape(2, 5, 2, 4)
                   for s in (1, 2, 3, 4))
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_CAUSAL)
    ref = torch_reference(q, k, v, dy, vis=visible_from_rules(MASK_CAUSAL, 5, 5)[None, None])
    for name in ("dq", "dk", "dv"):
        assert rel_err(r[name], ref[name]) < 1e-12


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("kind", ["none", "causal", "window", "bias"])
def test_finite_differences_of_forward_loss(kind):
    """Central differences of L = sum(dY * O), O from torch's forward, against the
    oracle's gradients (every entry of Q, K and V)."""
    B, H, Sq, Sk, D = 1, 1, 4, 5, 3
    q, k, v, dy = (_rand(s, 10 + n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                             (B, Sk, H, D), (B, Sq, H, D)]))
    bias = _rand((B, H, Sq, Sk), 20) if kind == "bias" else None
    mk = {"none": MASK_NONE, "causal": MASK_CAUSAL, "window": MASK_WINDOW, "bias": MASK_BIAS}[kind]
    vis = visible_from_rules(mk, Sq, Sk, 1)[None, None] if kind in ("causal", "window") else None
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))

    def loss(q_, k_, v_):
        with torch.no_grad():
            mask = torch.from_numpy(vis) if vis is not None else (
                torch.from_numpy(bias) if bias is not None else None)
            o = torch.nn.functional.scaled_dot_product_attention(
                _to_bhsd(q_), _to_bhsd(k_), _to_bhsd(v_), attn_mask=mask, scale=scale)
            return float((o * _to_bhsd(dy)).sum())

    r = oracle.attn_bwd(q, k, v, dy, mask_kind=mk, window=1, mask=bias)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            argm = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            fd[idx] = (loss(*args) - loss(*argm)) / (2 * h)
        assert rel_err(r[name], fd) < 1e-6, name


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("kind", [MASK_NONE, MASK_CAUSAL, MASK_WINDOW, MASK_BIAS])
def test_invariants(kind):
    B, H, Sq, Sk, D = 2, 3, 9, 13, 8
    q, k, v, dy = (_rand(s, 30 + n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                             (B, Sk, H, D), (B, Sq, H, D)]))
    bias = _rand((B, H, Sq, Sk), 40)
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=kind, window=3, mask=bias)
    # delta two ways: rowsum(P dP) and dY . O
    np.testing.assert_allclose(r["delta"], r["delta_o"], rtol=1e-12, atol=1e-12)
    for b in range(B):
        for h in range(H):
            dq, dk, dv = r["dq"][b, :, h], r["dk"][b, :, h], r["dv"][b, :, h]
            qq, kk, vv, gy = q[b, :, h], k[b, :, h], v[b, :, h], dy[b, :, h]
            # rowsum(dS) = 0 for every row  =>  sum_j dK_j = 0
            assert np.max(np.abs(dk.sum(0))) < 1e-12 * max(1, np.abs(dk).max())
            # S is bilinear in Q and K  =>  <dQ, Q> = <dK, K>
            assert abs((dq * qq).sum() - (dk * kk).sum()) < 1e-11
            # <dV, V> = sum_i delta_i = <dY, O>
            assert abs((dv * vv).sum() - r["delta"][b, h].sum()) < 1e-11
            # sum_j dV_j = sum over rows with a visible key of dY_i
            nonempty = r["l"][b, h] > 0
            np.testing.assert_allclose(dv.sum(0), gy[nonempty].sum(0), atol=1e-12)


def test_rowsum_ds_zero_per_row():
    """A constant feature K[..., 0] = 1 makes dQ_i[0] = sum_j dS_ij, which must be 0
    for every row (the scores only shift by a per-row constant)."""
    B, H, Sq, Sk, D = 1, 2, 7, 7, 6
    q, k, v, dy = (_rand(s, 50 + n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                             (B, Sk, H, D), (B, Sq, H, D)]))
    k[..., 0] = 1.0
    for kind in (MASK_NONE, MASK_CAUSAL, MASK_WINDOW):
        r = oracle.attn_bwd(q, k, v, dy, mask_kind=kind, window=2)
        assert np.max(np.abs(r["dq"][..., 0])) < 1e-13
        assert np.max(np.abs(r["dq"][..., 1:])) > 1e-3


def test_shift_invariance_of_keys_and_values():
    """K -> K + 1 c^T shifts each score row by a constant; V -> V + 1 c^T shifts O by c:
    neither changes any gradient."""
    B, H, Sq, Sk, D = 1, 2, 6, 9, 5
    q, k, v, dy = (_rand(s, 60 + n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                             (B, Sk, H, D), (B, Sq, H, D)]))
    c = _rand((D,), 70)
    r0 = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_CAUSAL)
    r1 = oracle.attn_bwd(q, k + c, v + c, dy, mask_kind=MASK_CAUSAL)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r1[name], r0[name], atol=1e-11)


# ---------------------------------------------------------------- closed forms
def test_single_key_closed_form():
    """Sk = 1: P = 1 for every row, so dS = 0: dQ = dK = 0 and dV = sum_i dY_i."""
    B, H, Sq, D = 2, 2, 5, 4
    q, k, v, dy = _rand((B, Sq, H, D), 1), _rand((B, 1, H, D), 2), _rand((B, 1, H, D), 3), \
        _rand((B, Sq, H, D), 4)
    for kind in (MASK_NONE, MASK_CAUSAL):
        r = oracle.attn_bwd(q, k, v, dy, mask_kind=kind)
        assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)
        np.testing.assert_allclose(r["dv"][:, 0], dy.sum(1), rtol=1e-14)


def test_window_zero_closed_form():
    """w = 0 (Sq = Sk): each query sees only its own key: dQ = dK = 0, dV_j = dY_j."""
    B, H, S, D = 1, 3, 6, 4
    q, k, v, dy = (_rand((B, S, H, D), n) for n in range(4))
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_WINDOW, window=0)
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)
    np.testing.assert_allclose(r["dv"], dy, rtol=1e-15)


def test_bias_with_zero_queries_is_softmax_of_bias():
    """Q = 0: scores equal the (unscaled) bias, so P_i = softmax(bias_i) and
    dV_j = sum_i softmax(bias_i)_j dY_i (scipy's softmax as the library routine)."""
    from scipy.special import softmax
    B, H, Sq, Sk, D = 1, 2, 4, 6, 3
    q = np.zeros((B, Sq, H, D))
    k, v, dy = _rand((B, Sk, H, D), 1), _rand((B, Sk, H, D), 2), _rand((B, Sq, H, D), 3)
    bias = _rand((B, H, Sq, Sk), 4) * 2
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_BIAS, mask=bias)
    for h in range(H):
        P = softmax(bias[0, h], axis=-1)
        np.testing.assert_allclose(r["dv"][0, :, h], P.T @ dy[0, :, h], rtol=1e-12)


def test_fully_masked_batch_is_zero():
    """Key padding that hides every key of batch 1: its rows have P = 0 and
    contribute nothing; batch 0 is unaffected."""
    B, H, Sq, Sk, D = 2, 2, 5, 7, 4
    q, k, v, dy = (_rand(s, n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                       (B, Sk, H, D), (B, Sq, H, D)]))
    valid = np.ones((B, 1, 1, Sk))
    valid[1] = 0.0
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_KEYPAD, mask=valid)
    for name in ("dq", "dk", "dv"):
        assert np.all(r[name][1] == 0.0)
    assert np.all(r["l"][1] == 0) and np.all(r["delta"][1] == 0) and np.all(r["m"][1] == -np.inf)
    r0 = oracle.attn_bwd(q[:1], k[:1], v[:1], dy[:1])
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r[name][0], r0[name][0], rtol=1e-15)


def test_causal_bottom_right_equals_padded_square_problem():
    """Queries at the last Sq of Sk positions: adding Sk - Sq leading query rows
    with dY = 0 to make a square causal problem changes no dK/dV (those rows have
    dP = 0 and delta = 0) and leaves the last rows' dQ unchanged.  The square
    problem is checked against torch's own is_causal=True."""
    B, H, Sq, Sk, D = 1, 2, 3, 8, 4
    q, k, v, dy = (_rand(s, 80 + n) for n, s in enumerate([(B, Sq, H, D), (B, Sk, H, D),
                                                             (B, Sk, H, D), (B, Sq, H, D)]))
    qpad = np.concatenate([_rand((B, Sk - Sq, H, D), 90), q], axis=1)
    dypad = np.concatenate([np.zeros((B, Sk - Sq, H, D)), dy], axis=1)
    r = oracle.attn_bwd(q, k, v, dy, mask_kind=MASK_CAUSAL)
    qt, kt, vt = (_to_bhsd(x).requires_grad_(True) for x in (qpad, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=float(np.float32(1) / np.sqrt(np.float32(D))))
    (o * _to_bhsd(dypad)).sum().backward()
    assert rel_err(r["dk"], _from_bhsd(kt.grad)) < 1e-12
    assert rel_err(r["dv"], _from_bhsd(vt.grad)) < 1e-12
    assert rel_err(r["dq"], _from_bhsd(qt.grad)[:, Sk - Sq:]) < 1e-12


def test_empty_dimensions():
    B, H, D = 1, 2, 4
    r = oracle.attn_bwd(np.zeros((B, 0, H, D)), _rand((B, 3, H, D), 1), _rand((B, 3, H, D), 2),
                        np.zeros((B, 0, H, D)))
    assert r["dk"].shape == (B, 3, H, D) and np.all(r["dk"] == 0) and np.all(r["dv"] == 0)
    r = oracle.attn_bwd(_rand((B, 3, H, D), 1), np.zeros((B, 0, H, D)), np.zeros((B, 0, H, D)),
                        _rand((B, 3, H, D), 2))
    assert np.all(r["dq"] == 0) and np.all(r["l"] == 0)


def test_rejects_bad_arguments():
    q = _rand((1, 2, 1, 4), 1)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, q, q, q, mask_kind=MASK_WINDOW, window=-1)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, q, q, q, mask_kind=7)


@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_gqa_matches_autograd(mask):
    """Grouped-query reference against torch float64 autograd of a forward whose
    query heads share K / V (gradients of a shared tensor sum by the chain rule)."""
    g = torch.Generator().manual_seed(77)
    B, Sq, Sk, H, Hkv, D = 2, 7, 9, 6, 2, 4
    q = torch.randn(B, Sq, H, D, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(B, Sk, Hkv, D, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(B, Sk, Hkv, D, generator=g, dtype=torch.float64, requires_grad=True)
    dy = torch.randn(B, Sq, H, D, generator=g, dtype=torch.float64)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    kk = k.repeat_interleave(H // Hkv, dim=2)
    vv = v.repeat_interleave(H // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) * scale
    off = max(Sk - Sq, 0)
    i = torch.arange(Sq)[:, None] + off
    j = torch.arange(Sk)[None, :]
    if mask == "causal":
        s = s.masked_fill(j > i, float("-inf"))
    elif mask == "window":
        s = s.masked_fill((j > i) | (j < i - 3), float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vv)
    o.backward(dy)
    code = {"none": oracle.MASK_NONE, "causal": oracle.MASK_CAUSAL, "window": oracle.MASK_WINDOW}[mask]
    r = oracle.attn_bwd_gqa(q.detach(), k.detach(), v.detach(), dy, mask_kind=code, window=3)
    np.testing.assert_allclose(r["dq"], q.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dk"], k.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dv"], v.grad.numpy(), rtol=1e-11, atol=1e-12)
