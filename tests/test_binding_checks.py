"""Host-side checks of the Python binding: tensors that cannot be handed to the
C ABI (host memory, mixed dtypes, wrong shapes, a non-contiguous last axis, a
mask that is not float32) are rejected with ValueError before any pointer is
taken or anything is launched.  No GPU is needed: every case fails in Python.

The dtype and shape checks come before the device check, so each of them is
reachable with CPU tensors; the device check itself is exercised by consistent
CPU tensors, which must never reach the library."""
import numpy as np
import pytest
import torch

import scaled_dot_product_bwd_amd as sdb


def _dense(B=1, Sq=8, Sk=8, H=2, Hkv=2, D=32, dtype=torch.bfloat16):
    q = torch.zeros(B, Sq, H, D, dtype=dtype)
    k = torch.zeros(B, Sk, Hkv, D, dtype=dtype)
    return q, k, k.clone(), q.clone()


def test_host_tensors_are_rejected_before_any_launch():
    q, k, v, dy = _dense()
    with pytest.raises(ValueError, match="CUDA"):
        sdb.attn_bwd(q, k, v, dy)
    with pytest.raises(ValueError, match="CUDA"):
        sdb.make_args(q, k, v, dy)


@pytest.mark.parametrize("which", ["k", "v", "dy"])
def test_mixed_dtypes_are_rejected(which):
    q, k, v, dy = _dense(dtype=torch.float32)
    t = {"k": k, "v": v, "dy": dy}
    t[which] = t[which].to(torch.bfloat16)
    with pytest.raises(ValueError, match=which + " is torch.bfloat16"):
        sdb.attn_bwd(q, t["k"], t["v"], t["dy"])


def test_unsupported_dtype_is_rejected():
    q, k, v, dy = (x.to(torch.float16) for x in _dense())
    with pytest.raises(ValueError, match="float32 or bfloat16"):
        sdb.attn_bwd(q, k, v, dy)


def test_output_dtype_and_shape_are_checked():
    q, k, v, dy = _dense()
    with pytest.raises(ValueError, match="dk is torch.float32"):
        sdb.attn_bwd(q, k, v, dy, out=(q.clone(), k.float(), v.clone()))
    with pytest.raises(ValueError, match="dq has shape"):
        sdb.attn_bwd(q, k, v, dy, out=(q[:, :4].clone(), k.clone(), v.clone()))


def test_mask_must_be_float32_and_broadcast():
    q, k, v, dy = _dense(dtype=torch.float32)
    with pytest.raises(ValueError, match="mask is torch.float64"):
        sdb.attn_bwd(q, k, v, dy, mask_kind="keypad", mask=torch.ones(1, 1, 1, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="does not broadcast"):
        sdb.attn_bwd(q, k, v, dy, mask_kind="bias", mask=torch.zeros(1, 3, 8, 8))


def test_shape_mismatches_are_rejected():
    q, k, v, dy = _dense()
    with pytest.raises(ValueError, match="v has shape"):
        sdb.attn_bwd(q, k, v[:, :5].clone(), dy)
    with pytest.raises(ValueError, match="dy has shape"):
        sdb.attn_bwd(q, k, v, dy[..., :16].clone())
    with pytest.raises(ValueError, match=r"\[B, S, H, D\]"):
        sdb.attn_bwd(q[0], k, v, dy)


def test_last_axis_must_be_contiguous():
    q, k, v, dy = _dense(D=32, Sk=32)
    kt = k.transpose(1, 3)  # [B, D, H, S] viewed as [B, S', H, D'] with stride(-1) != 1
    with pytest.raises(ValueError, match="contiguous last axis"):
        sdb.attn_bwd(q, kt, kt, dy)


def test_forward_statistics_are_checked():
    q, k, v, dy = _dense(dtype=torch.float32)
    with pytest.raises(ValueError, match="go together"):
        sdb.attn_bwd(q, k, v, dy, fwd_lse=torch.zeros(1, 2, 8))
    with pytest.raises(ValueError, match="fwd_lse has shape"):
        sdb.attn_bwd(q, k, v, dy, fwd_lse=torch.zeros(2, 8), fwd_out=q.clone())
    with pytest.raises(ValueError, match="fwd_out is torch.bfloat16"):
        sdb.attn_bwd(q, k, v, dy, fwd_lse=torch.zeros(1, 2, 8), fwd_out=q.bfloat16())


def _paged(dtype=torch.bfloat16, nq=4, heads=4, kvh=2, D=32, slots=32):
    plan = sdb.paged_plan(np.array([16, 9]), np.array([[0], [1]]), np.array([0, 0, 1, 1]),
                          np.array([14, 15, 7, 8]), heads=heads, kv_heads=kvh, page_size=16,
                          pool_pages=2)
    q = torch.zeros(nq, heads, D, dtype=dtype)
    pool = torch.zeros(slots, kvh, D, dtype=dtype)
    stats = torch.zeros(nq, heads, 3)
    return plan, q, pool, stats


def test_paged_host_tensors_are_rejected():
    plan, q, pool, stats = _paged()
    plan.device_words = torch.from_numpy(plan.words)  # a host copy: must not reach a kernel
    with pytest.raises(ValueError, match="CUDA"):
        sdb.attn_bwd_paged(q, q.clone(), pool, pool.clone(), stats, plan)
    with pytest.raises(ValueError, match="CUDA"):
        sdb.make_paged_args(q, q.clone(), pool, pool.clone(), stats, plan)


def test_paged_dtype_and_shape_checks():
    plan, q, pool, stats = _paged()
    with pytest.raises(ValueError, match="stats is torch.bfloat16"):
        sdb.attn_bwd_paged(q, q.clone(), pool, pool.clone(), stats.bfloat16(), plan)
    with pytest.raises(ValueError, match="v_pool is torch.float32"):
        sdb.attn_bwd_paged(q, q.clone(), pool, pool.float(), stats, plan)
    with pytest.raises(ValueError, match="dy has shape"):
        sdb.attn_bwd_paged(q, q[:2].clone(), pool, pool.clone(), stats, plan)
    with pytest.raises(ValueError, match="dk_pool has shape"):
        sdb.attn_bwd_paged(q, q.clone(), pool, pool.clone(), stats, plan, dk_pool=pool[:16].clone())
    with pytest.raises(ValueError, match="must be contiguous"):
        wide = torch.zeros(32, 2, 64, dtype=torch.bfloat16)[:, :, :32]
        sdb.attn_bwd_paged(q, q.clone(), wide, pool.clone(), stats, plan)


def test_paged_query_side_and_latent_checks():
    plan, q, pool, stats = _paged()
    with pytest.raises(ValueError, match="out is torch.bfloat16"):
        sdb.paged_row_stats(q, q.clone(), pool, pool.clone(), plan, out=stats.bfloat16())
    qp = torch.zeros(4, 4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kp_pool has shape"):
        sdb.attn_bwd_paged_mla(q, qp, q.clone(), pool, torch.zeros(32, 2, 32, dtype=torch.bfloat16),
                               stats, plan)
