"""attn_bwd_noalloc (the dense backward with its row statistics in the
library's static per-GPU scratch) against attn_bwd (the same backward on a
torch-allocated workspace), through the C ABI.

Two calls in a row, the second smaller than the first and in another dtype and
mask, so the second runs on scratch the first left filled: each must give
attn_bwd's bits.  The call itself allocates nothing (torch's allocator count is
unchanged across it).  Sizes past the scratch are refused on the host before
any HIP call.
"""
import ctypes

import pytest
import torch

import sdpa_inputs
import scaled_dot_product_bwd_amd as sdb
from scaled_dot_product_bwd_amd import _abi

# (B, H, S, D, dtype, mask, window, seed): a larger call, then a smaller one.
CASES = [
    (2, 4, 700, 128, torch.bfloat16, "causal", 0, 31),
    (1, 2, 300, 64, torch.float32, "window", 40, 32),
]


@pytest.mark.gpu
def test_noalloc_equals_attn_bwd_on_two_calls_in_a_row():
    lib = sdb.load_library()
    dev = torch.device("cuda:0")
    for B, H, S, D, dtype, mask, window, seed in CASES:
        q, k, v, dy, _ = sdpa_inputs.dense_inputs(B, S, S, H, D, seed=seed, dtype=dtype)
        qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dy))
        # the reference on a workspace of exactly the statistics planes: the
        # form attn_bwd_noalloc runs (a split-sized workspace would give the
        # split form, equal only up to rounding)
        ws = torch.empty(sdb.workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
        ref = sdb.attn_bwd(qd, kd, vd, gd, mask_kind=mask, window=window, workspace=ws)
        outs = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
        args = sdb.make_args(qd, kd, vd, gd, *outs, mask_kind=mask, window=window)
        assert not args.workspace  # no workspace is passed: the scratch is used
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        rc = lib.attn_bwd_noalloc(ctypes.byref(args),
                                  ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        assert rc == _abi.ATTN_OK, lib.attn_bwd_last_error().decode()
        assert torch.cuda.memory_allocated(dev) == before
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, want), (name, B, H, S, D, dtype, mask)


def test_noalloc_refuses_sizes_past_the_scratch_before_any_hip_call():
    lib = sdb.load_library()
    a = _abi.AttnBwdArgs()
    a.dtype, a.wrt, a.D, a.scale = _abi.ATTN_BF16, _abi.ATTN_WRT_ALL, 128, 0.088
    a.B, a.H, a.Sq, a.Sk = 1, 1, (1 << 20) + 1, 64
    assert lib.attn_bwd_noalloc(ctypes.byref(a), None) == _abi.ATTN_E_WORKSPACE
    assert b"at most 1048576 rows" in lib.attn_bwd_last_error()
    a.B, a.H, a.Sq = 2 ** 40, 2 ** 40, 2
    assert lib.attn_bwd_noalloc(ctypes.byref(a), None) == _abi.ATTN_E_WORKSPACE
    a.B = -1
    assert lib.attn_bwd_noalloc(ctypes.byref(a), None) == _abi.ATTN_E_INVALID
