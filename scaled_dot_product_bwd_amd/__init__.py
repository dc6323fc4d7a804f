"""MI355X (gfx950) scaled dot-product attention backward.

A thin ctypes binding over ``libattn_bwd.so`` (C ABI in ``include/attn_bwd.h``).
This module only marshals arguments: torch supplies device memory and the
current stream, and every step of the computation runs in the HIP kernels.
There is no CPU fallback: without the built library every call raises.

    dq, dk, dv = attn_bwd(q, k, v, dy, mask_kind="causal")

    plan = paged_plan(seq_lens, block_table, query_seq, query_pos, heads=32,
                      kv_heads=8, page_size=16, pool_pages=N, device="cuda")
    stats, dq = paged_stats_dq(q, dy, k_pool, v_pool, plan)
    attn_bwd_paged(q, dy, k_pool, v_pool, stats, plan, dk_pool=dk, dv_pool=dv)

Tensors are ``[B, S, H, D]`` (any strides with ``D`` contiguous; pass
``x.transpose(1, 2)`` for a ``[B, H, S, D]`` tensor), float32 or bfloat16, on the
GPU.  The semantics are those of rlx-cpu 0.2.17 src/attention_bwd.rs
(`attention_backward_all`) with the mask codes of rlx-wgpu 0.2.1
attention_bwd.wgsl (`mask_score`); the paged path is ruDNN 0.1.43
src/paged_attention/ordered_kernel.rs (`history_backward`).
"""
from __future__ import annotations

import ctypes
import math
import os

from . import _abi
from ._abi import (ATTN_BF16, ATTN_F32, ATTN_MASK_BIAS, ATTN_MASK_CAUSAL,
                   ATTN_MASK_FLAG_CAUSAL, ATTN_MASK_KEYPAD, ATTN_MASK_NONE, ATTN_MASK_WINDOW,
                   ATTN_WRT_ALL, ATTN_WRT_K, ATTN_WRT_Q, ATTN_WRT_V, AttnBwdArgs,
                   AttnBwdPagedArgs, AttnError, load_library, library_path)

__all__ = ["attn_bwd", "attn_bwd_noalloc", "attn_bwd_stage", "workspace_bytes",
           "split_workspace_bytes", "make_args", "AttnError",
           "load_library", "library_path", "MASKS", "WRT", "PagedPlan", "paged_plan",
           "attn_bwd_paged", "attn_bwd_paged_mla", "make_paged_args", "paged_row_stats",
           "paged_q_workspace",
           "attn_bwd_paged_dq", "paged_stats_dq"]

MASKS = {"none": ATTN_MASK_NONE, "causal": ATTN_MASK_CAUSAL, "keypad": ATTN_MASK_KEYPAD,
         "window": ATTN_MASK_WINDOW, "bias": ATTN_MASK_BIAS}
WRT = {"q": ATTN_WRT_Q, "k": ATTN_WRT_K, "v": ATTN_WRT_V, "all": ATTN_WRT_ALL}


def _torch():
    import torch
    return torch


def workspace_bytes(B: int, H: int, Sq: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, Sq))


def split_workspace_bytes(B: int, H: int, Sq: int, Sk: int, D: int) -> int:
    """The workspace size that also enables the split form of the
    query-major passes (attn_bwd_split_workspace_bytes)."""
    return int(load_library().attn_bwd_split_workspace_bytes(B, H, Sq, Sk, D))


def _strides3(t):
    s = t.stride()
    return (s[0], s[1], s[2])


# ---------------------------------------------------------------------------
# Argument checks on the torch side.  The C ABI takes raw pointers and cannot
# tell a host address from a device one, nor see a tensor's dtype: a CPU tensor
# or a mismatched dtype would reach a kernel as a wild pointer or a buffer read
# past its end.  So every tensor is checked here, before its pointer is taken:
# dtype and shape first, then the device (all on q's GPU).

def _fail(msg):
    raise ValueError(msg)


def _check_float(name, t, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        _fail(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        _fail(f"{name} is {t.dtype}, expected {dtype}")


def _check_rows(name, t, shape):
    """t has exactly `shape` and a contiguous last axis (the kernels read D
    contiguous elements per row and are given only the outer strides)."""
    if tuple(t.shape) != tuple(shape):
        _fail(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        _fail(f"{name} must have a contiguous last axis (stride {t.stride(-1)})")


def _check_devices(ref_device, named):
    if ref_device.type != "cuda":
        _fail(f"tensors must be on a CUDA (HIP) device, got {ref_device}")
    for name, t in named:
        if t is not None and t.device != ref_device:
            _fail(f"{name} is on {t.device}, expected {ref_device} (the device of q)")


def _io_dtype(q):
    torch = _torch()
    if not isinstance(q, torch.Tensor):
        _fail(f"q must be a torch.Tensor, got {type(q).__name__}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        _fail(f"q is {q.dtype}: the kernels take float32 or bfloat16")
    return q.dtype


def check_dense_tensors(q, k, v, dy, dq=None, dk=None, dv=None, mask=None, workspace=None,
                        fwd_lse=None, fwd_out=None):
    """Raises ValueError unless the tensors fit one dense call: q, dy
    [B, Sq, H, D]; k, v [B, Sk, Hkv, D] (H a multiple of Hkv); outputs shaped
    like their inputs; all of q's dtype (float32 or bfloat16) with a contiguous
    last axis; mask float32 broadcastable to [B, H, Sq, Sk]; fwd_lse float32
    [B, H, Sq]; fwd_out like q; everything on q's GPU."""
    torch = _torch()
    dt = _io_dtype(q)
    if q.dim() != 4:
        _fail(f"q must be [B, S, H, D], got {q.dim()} dims")
    B, Sq, H, D = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        _fail("k must be a [B, S, H, D] tensor")
    Sk, Hkv = k.shape[1], k.shape[2]
    named = [("q", q), ("k", k), ("v", v), ("dy", dy), ("dq", dq), ("dk", dk), ("dv", dv)]
    shapes = {"q": (B, Sq, H, D), "dy": (B, Sq, H, D), "dq": (B, Sq, H, D),
              "k": (B, Sk, Hkv, D), "v": (B, Sk, Hkv, D), "dk": (B, Sk, Hkv, D),
              "dv": (B, Sk, Hkv, D)}
    for name, t in named:
        if t is None and name in ("q", "k", "v", "dy"):
            _fail(f"{name} is required")
        if t is not None:
            _check_float(name, t, dt)
            _check_rows(name, t, shapes[name])
    if mask is not None:
        _check_float("mask", mask, torch.float32)
        try:
            torch.broadcast_shapes(tuple(mask.shape), (B, H, Sq, Sk))
        except RuntimeError:
            _fail(f"mask of shape {tuple(mask.shape)} does not broadcast to {(B, H, Sq, Sk)}")
    if fwd_lse is not None:
        _check_float("fwd_lse", fwd_lse, torch.float32)
        if tuple(fwd_lse.shape) != (B, H, Sq):
            _fail(f"fwd_lse has shape {tuple(fwd_lse.shape)}, expected {(B, H, Sq)}")
    if fwd_out is not None:
        _check_float("fwd_out", fwd_out, dt)
        _check_rows("fwd_out", fwd_out, (B, Sq, H, D))
    if workspace is not None and not isinstance(workspace, torch.Tensor):
        _fail("workspace must be a torch.Tensor")
    _check_devices(q.device, named + [("mask", mask), ("workspace", workspace),
                                      ("fwd_lse", fwd_lse), ("fwd_out", fwd_out)])


def check_paged_tensors(q, dy, k_pool, v_pool, stats, plan, dk_pool=None, dv_pool=None, *,
                        qp=None, kp_pool=None, dkp_pool=None, outs=()):
    """Raises ValueError unless the tensors fit one paged call: q, dy
    [nq, heads, D]; pools [slots, kv_heads, D] (gradient pools shaped like
    them); stats float32 [nq, heads, 3]; latent position parts qp
    [nq, heads, P], kp_pool / dkp_pool [slots, kv_heads, P]; all contiguous, of
    q's dtype (float32 or bfloat16) except stats, on q's GPU, where the plan's
    device copy must live too.  outs: extra (name, tensor, shape, dtype)
    outputs (the query side's statistics or dQ)."""
    torch = _torch()
    dt = _io_dtype(q)
    if q.dim() != 3:
        _fail(f"q must be [nq, heads, D], got {q.dim()} dims")
    nq, heads, D = q.shape
    if not isinstance(k_pool, torch.Tensor) or k_pool.dim() != 3:
        _fail("k_pool must be a [slots, kv_heads, D] tensor")
    slots, kvh = k_pool.shape[0], k_pool.shape[1]
    named = [("q", q, (nq, heads, D), dt), ("dy", dy, (nq, heads, D), dt),
             ("k_pool", k_pool, (slots, kvh, D), dt), ("v_pool", v_pool, (slots, kvh, D), dt),
             ("stats", stats, (nq, heads, 3), torch.float32),
             ("dk_pool", dk_pool, (slots, kvh, D), dt), ("dv_pool", dv_pool, (slots, kvh, D), dt)]
    if qp is not None:
        P = qp.shape[-1] if qp.dim() == 3 else -1
        named += [("qp", qp, (nq, heads, P), dt), ("kp_pool", kp_pool, (slots, kvh, P), dt),
                  ("dkp_pool", dkp_pool, (slots, kvh, P), dt)]
    named += list(outs)
    for name, t, shape, want in named:
        if t is None:
            if name in ("q", "dy", "k_pool", "stats"):
                _fail(f"{name} is required")
            continue
        _check_float(name, t, want)
        _check_rows(name, t, shape)
        if not t.is_contiguous():
            _fail(f"{name} must be contiguous")
    if plan.device_words is not None and plan.device_words.device != q.device:
        _fail(f"the plan was uploaded to {plan.device_words.device}, expected {q.device}")
    _check_devices(q.device, [(n, t) for n, t, _, _ in named])


# ---------------------------------------------------------------------------
# Streams.  Work is enqueued on the caller's stream (default: the current one).
# When that is another stream, it first waits for the current stream (where the
# binding allocated, filled, copied or uploaded what the call reads), and every
# tensor the binding created for the call is recorded on it, so torch's caching
# allocator does not hand that memory to later work on the current stream while
# the kernels may still run.

def _launch_stream(stream, device):
    """(void* handle, side) -- side is the caller's stream when it is not the
    current one, else None."""
    torch = _torch()
    cur = torch.cuda.current_stream(device)
    if stream is None or stream == cur:
        return ctypes.c_void_p(cur.cuda_stream), None
    stream.wait_stream(cur)
    return ctypes.c_void_p(stream.cuda_stream), stream


def _record(side, *tensors):
    if side is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(side)


def make_args(q, k, v, dy, dq=None, dk=None, dv=None, *, wrt="all", mask_kind="none",
              causal=False, window=0, mask=None, threshold=0.5, scale=None, workspace=None):
    """Builds the attn_bwd_args struct for already-allocated tensors.  The
    tensors are checked here (check_dense_tensors: dtype, shape, device); sizes,
    strides, alignment and aliasing are validated by the library."""
    torch = _torch()
    check_dense_tensors(q, k, v, dy, dq, dk, dv, mask=mask, workspace=workspace)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    a = AttnBwdArgs()
    a.dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F32
    a.wrt = WRT[wrt] if isinstance(wrt, str) else int(wrt)
    a.B, a.H, a.Sq, a.Sk, a.D = B, H, Sq, Sk, D
    a.Hkv = k.shape[2]  # grouped-query attention when k has fewer heads than q
    a.q, a.k, a.v, a.dy = q.data_ptr(), k.data_ptr(), v.data_ptr(), dy.data_ptr()
    a.q_stride[:], a.k_stride[:] = _strides3(q), _strides3(k)
    a.v_stride[:], a.dy_stride[:] = _strides3(v), _strides3(dy)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            setattr(a, name, t.data_ptr())
            getattr(a, name + "_stride")[:] = _strides3(t)
    a.mask_kind = MASKS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    a.mask_flags = ATTN_MASK_FLAG_CAUSAL if causal else 0
    a.window = int(window or 0)
    if mask is not None:
        mv = mask.expand(B, H, Sq, Sk)
        a.mask = mv.data_ptr()
        a.mask_stride[:] = mv.stride()
    a.mask_threshold = float(threshold)
    a.scale = float(scale) if scale is not None else float(
        torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def _check(rc):
    if rc != 0:
        msg = load_library().attn_bwd_last_error().decode(errors="replace")
        raise AttnError(rc, msg)


def _stream_handle(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def attn_bwd_stage(stage: str, args: AttnBwdArgs, stream=None):
    """Runs one stage ("all", "row_stats", "kv", "dq" or "stats_dq") of the
    backward on the given (default: current) torch stream.  The tensors behind
    `args` belong to the caller, who keeps them alive (and, on a side stream,
    ordered) until the stream has passed this call."""
    lib = load_library()
    fn = {"all": lib.attn_bwd, "row_stats": lib.attn_bwd_row_stats, "kv": lib.attn_bwd_kv,
          "dq": lib.attn_bwd_dq, "stats_dq": lib.attn_bwd_stats_dq}[stage]
    _check(fn(ctypes.byref(args), _stream_handle(stream)))


def attn_bwd(q, k, v, dy, *, wrt="all", mask_kind="none", causal=False, window=0, mask=None,
             threshold=0.5, scale=None, out=None, workspace=None, stream=None,
             return_workspace=False, fwd_lse=None, fwd_out=None):
    """Gradients of scaled dot-product attention.  k and v may have fewer heads
    than q (grouped-query attention: H a multiple of Hkv, query head h reads
    K / V head h // (H // Hkv)); dk and dv then have Hkv heads.

    mask_kind: "none", "causal", "keypad" (mask = key validity, hidden iff
    < threshold), "window" (keeps [a - window, a] for query position a) or
    "bias" (mask added to the scaled scores); ``causal=True`` adds the causal
    rule to "keypad" / "bias".  ``mask`` is float32 and broadcasts to
    [B, H, Sq, Sk] ([B, 1, 1, Sk] for per-batch padding).
    With ``fwd_lse`` (float32 [B, H, Sq]: the forward's natural log-sum-exp
    per row) and ``fwd_out`` (the forward output O, like q), the row
    statistics come from them (attn_bwd_from_forward) instead of a recompute.
    Returns (dq, dk, dv); entries that ``wrt`` does not ask for are None.
    """
    torch = _torch()
    if fwd_lse is not None or fwd_out is not None:
        if fwd_lse is None or fwd_out is None:
            raise ValueError("fwd_lse and fwd_out go together")
    check_dense_tensors(q, k, v, dy, *(out if out is not None else (None, None, None)),
                        mask=mask, workspace=workspace, fwd_lse=fwd_lse, fwd_out=fwd_out)
    B, Sq, H, D = q.shape
    w = WRT[wrt] if isinstance(wrt, str) else int(wrt)
    if out is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format) if w in (ATTN_WRT_Q, ATTN_WRT_ALL) else None
        dk = torch.empty_like(k, memory_format=torch.contiguous_format) if w in (ATTN_WRT_K, ATTN_WRT_ALL) else None
        dv = torch.empty_like(v, memory_format=torch.contiguous_format) if w in (ATTN_WRT_V, ATTN_WRT_ALL) else None
    else:
        dq, dk, dv = out
    if workspace is None:
        nbytes = workspace_bytes(B, H, Sq)
        # the split form of the passes pays when a pass's workgroups (per
        # query block and head, or per key block and K / V head) fill at most
        # half of the GPU (the library decides; a larger workspace only makes
        # it possible)
        blocks = min(B * H * ((Sq + 127) // 128), B * k.shape[2] * ((k.shape[1] + 127) // 128))
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        if 2 * blocks <= cus:
            nbytes = max(nbytes, split_workspace_bytes(B, H, Sq, k.shape[1], D))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = make_args(q, k, v, dy, dq, dk, dv, wrt=w, mask_kind=mask_kind, causal=causal,
                     window=window, mask=mask, threshold=threshold, scale=scale,
                     workspace=workspace)
    lse = fwd_lse.contiguous() if fwd_lse is not None else None
    handle, side = _launch_stream(stream, q.device)
    if fwd_lse is not None:
        ost = (ctypes.c_int64 * 3)(*_strides3(fwd_out))
        _check(load_library().attn_bwd_from_forward(
            ctypes.byref(args), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(fwd_out.data_ptr()),
            ost, handle))
    else:
        _check(load_library().attn_bwd(ctypes.byref(args), handle))
    _record(side, dq, dk, dv, workspace, lse)
    if return_workspace:
        return (dq, dk, dv), workspace
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, dy, *, out, wrt="all", mask_kind="none", causal=False, window=0,
                     mask=None, threshold=0.5, scale=None, stream=None):
    """attn_bwd without any device allocation (attn_bwd_noalloc): the caller
    passes the outputs ``out = (dq, dk, dv)`` (None where ``wrt`` does not ask
    for one) and the row statistics live in the library's static per-GPU
    scratch (B * H * Sq at most 2^20 rows).  Calls that overlap on one GPU
    race on that scratch.  Returns ``out``."""
    dq, dk, dv = out
    args = make_args(q, k, v, dy, dq, dk, dv, wrt=wrt, mask_kind=mask_kind, causal=causal,
                     window=window, mask=mask, threshold=threshold, scale=scale)
    handle, _ = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_noalloc(ctypes.byref(args), handle))
    return dq, dk, dv


def row_stats_views(workspace, B, H, Sq):
    """(m, l, delta) as float32 views [B, H, Sq] of a workspace filled by attn_bwd."""
    plane = ((B * H * Sq * 4 + 255) // 256) * 256
    f = workspace.view(_torch().uint8)
    out = []
    for i in range(3):
        out.append(f[i * plane: i * plane + B * H * Sq * 4].view(_torch().float32).view(B, H, Sq))
    return tuple(out)


# ---------------------------------------------------------------------------
# Paged history backward.

class PagedPlan:
    """Host plan words (numpy int32) and, once uploaded, their device copy."""

    def __init__(self, words, *, heads, kv_heads, page_size, pool_pages, nq, device=None):
        self.words = words
        self.heads, self.kv_heads, self.page_size = heads, kv_heads, page_size
        self.pool_pages, self.nq = pool_pages, nq
        self.device_words = None
        if device is not None:
            self.to(device)

    def to(self, device):
        torch = _torch()
        self.device_words = torch.from_numpy(self.words).to(device)
        return self

    def header(self, w):
        return int(self.words[w])

    @property
    def items(self):
        return self.header(_abi.W_ITEMS)

    def _table(self, off_word, n):
        off = self.header(off_word)
        return self.words[off: off + n]

    def listed_pages(self):
        """Physical pages whose slots the backward writes, ascending."""
        return self._table(_abi.W_OFF_LISTED, self.header(_abi.W_LISTED)).copy()

    def item_slots(self):
        """[items, 128] slot entries (slot * 2 + live, -1 = unused lane)."""
        return self._table(_abi.W_OFF_ITEM_SLOTS,
                           self.items * _abi.PLAN_ITEM_SLOTS).reshape(self.items, -1).copy()


def _np_i32(x):
    import numpy as np
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def paged_plan(seq_lens, block_table, query_seq, query_pos, *, heads, kv_heads, page_size,
               pool_pages, device=None):
    """Builds the host plan of the paged backward (attn_bwd_paged_plan_build) and,
    with ``device``, uploads it.  seq_lens [nseq], block_table [nseq, max_pages],
    query_seq / query_pos [nq]: integer arrays or tensors (any device)."""
    import numpy as np
    lib = load_library()
    lens = _np_i32(seq_lens).reshape(-1)
    bt = _np_i32(block_table)
    nseq = int(lens.size)
    bt = bt.reshape(nseq, -1) if bt.size else np.zeros((nseq, 0), np.int32)
    qs = _np_i32(query_seq).reshape(-1)
    qp = _np_i32(query_pos).reshape(-1)
    nq = int(qs.size)
    vp = ctypes.c_void_p
    words = lib.attn_bwd_paged_plan_words(nseq, lens.ctypes.data_as(vp), bt.shape[1], nq, heads,
                                          kv_heads, page_size, pool_pages)
    if words < 0:
        _check(_abi.ATTN_E_INVALID)
    buf = np.zeros(max(int(words), 32), dtype=np.int32)
    _check(lib.attn_bwd_paged_plan_build(
        nseq, lens.ctypes.data_as(vp), bt.ctypes.data_as(vp), bt.shape[1], nq,
        qs.ctypes.data_as(vp), qp.ctypes.data_as(vp), heads, kv_heads, page_size, pool_pages,
        buf.ctypes.data_as(vp), buf.size))
    used = int(buf[_abi.W_WORDS])
    return PagedPlan(buf[:used].copy(), heads=heads, kv_heads=kv_heads, page_size=page_size,
                     pool_pages=pool_pages, nq=nq, device=device)


def make_paged_args(q, dy, k_pool, v_pool, stats, plan, dk_pool=None, dv_pool=None, *,
                    causal=True, scale=None, need=3, outs=(), kv_workgroups=0):
    """Builds the attn_bwd_paged_args struct; the tensors are checked first
    (check_paged_tensors), the plan must already be on q's device.
    kv_workgroups: 0 lets the library pick the dK / dV kernel form; n > 0
    forces the persistent form with n workgroups, -1 one workgroup per
    (item, KV head) unit (bf16, not latent; every form gives identical bits)."""
    torch = _torch()
    if plan.device_words is None:
        raise ValueError("the plan has no device copy: call plan.to(device) first")
    check_paged_tensors(q, dy, k_pool, v_pool, stats, plan, dk_pool, dv_pool, outs=outs)
    nq, heads, D = q.shape
    a = AttnBwdPagedArgs()
    a.dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F32
    a.need = int(need)
    a.heads, a.kv_heads, a.head_dim = heads, k_pool.shape[1], D
    a.page_size, a.causal = plan.page_size, int(bool(causal))
    a.nq, a.pool_pages = nq, plan.pool_pages
    a.scale = float(scale) if scale is not None else float(
        torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    a.q, a.dy = q.data_ptr(), dy.data_ptr()
    a.k_pool, a.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
    a.stats = stats.data_ptr()
    a.plan_host = plan.words.ctypes.data
    a.plan = plan.device_words.data_ptr()
    if dk_pool is not None:
        a.dk_pool = dk_pool.data_ptr()
    if dv_pool is not None:
        a.dv_pool = dv_pool.data_ptr()
    a.kv_workgroups = int(kv_workgroups)
    return a


def attn_bwd_paged(q, dy, k_pool, v_pool, stats, plan, *, dk_pool=None, dv_pool=None,
                   need="dkdv", causal=True, scale=None, stream=None, kv_workgroups=0):
    """dK / dV of the paged grouped-query history backward, written into the
    given gradient pools at the slots of listed pages (other slots untouched);
    pools that are not given are allocated zero-filled.  q, dy: [nq, heads, D];
    pools: [pool_pages * page_size, kv_heads, D] (contiguous, fp32 or bf16, on
    the GPU); stats: float32 [nq, heads, 3] = (max, denominator, delta); plan:
    a PagedPlan uploaded to the same device.  kv_workgroups: see
    make_paged_args.  Returns (dk_pool, dv_pool)."""
    torch = _torch()
    n = {"dk": 1, "dv": 2, "dkdv": 3}[need] if isinstance(need, str) else int(need)
    check_paged_tensors(q, dy, k_pool, v_pool, stats, plan, dk_pool, dv_pool)
    if plan.device_words is None:
        plan.to(q.device)
    if dk_pool is None and n & 1:
        dk_pool = torch.zeros_like(k_pool)
    if dv_pool is None and n & 2:
        dv_pool = torch.zeros_like(v_pool)
    args = make_paged_args(q, dy, k_pool, v_pool, stats, plan, dk_pool, dv_pool,
                           causal=causal, scale=scale, need=n, kv_workgroups=kv_workgroups)
    handle, side = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_paged(ctypes.byref(args), handle))
    _record(side, dk_pool, dv_pool, plan.device_words)
    return dk_pool, dv_pool


def attn_bwd_paged_mla(q, qp, dy, latent_pool, kp_pool, stats, plan, *, dlat_pool=None,
                       dkp_pool=None, need="both", causal=True, scale=None, stream=None):
    """Latent (MLA) variant of attn_bwd_paged: each slot's latent row is both its
    key and its value, and a position key adds qp . kp to the score.
    q, dy: [nq, heads, D]; qp: [nq, heads, P]; latent_pool: [slots, kv_heads, D];
    kp_pool: [slots, kv_heads, P] (D in {64, 128}, for bf16 also {192, 256};
    P in {0, 32, 64}).  Writes the latent's gradient (ds q + p dY, summed) into
    dlat_pool and the position keys' (ds qp) into dkp_pool at the slots of
    listed pages; pools that are not given are allocated zero-filled.  The default scale is 1/sqrt(D + P).
    need: "dlat", "dkp" or "both".  Returns (dlat_pool, dkp_pool)."""
    torch = _torch()
    n = {"dlat": 1, "dkp": 4, "both": 5}[need] if isinstance(need, str) else int(need)
    check_paged_tensors(q, dy, latent_pool, latent_pool, stats, plan, dlat_pool, None, qp=qp,
                        kp_pool=kp_pool, dkp_pool=dkp_pool)
    D, P = q.shape[2], qp.shape[2]
    if P == 0:
        n &= 1
    if plan.device_words is None:
        plan.to(q.device)
    if dlat_pool is None and n & 1:
        dlat_pool = torch.zeros_like(latent_pool)
    if dkp_pool is None and n & 4:
        dkp_pool = torch.zeros_like(kp_pool)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(D + P), dtype=torch.float32))
    args = make_paged_args(q, dy, latent_pool, latent_pool, stats, plan, dlat_pool, None,
                           causal=causal, scale=scale, need=n)
    args.v_pool = None
    args.mla, args.position_dim = 1, P
    args.qp = qp.data_ptr() if qp.numel() else None
    args.kp_pool = kp_pool.data_ptr() if kp_pool.numel() else None
    if dkp_pool is not None:
        args.dkp_pool = dkp_pool.data_ptr()
    handle, side = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_paged(ctypes.byref(args), handle))
    _record(side, dlat_pool, dkp_pool, plan.device_words)
    return dlat_pool, dkp_pool


def paged_q_workspace(plan, head_dim, device):
    """A device workspace for the split form of the query side (torch-allocated)."""
    torch = _torch()
    n = load_library().attn_bwd_paged_q_workspace_bytes(plan.words.ctypes.data, int(head_dim))
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def _set_q_workspace(args, ws):
    if ws is not None:
        args.q_workspace = ws.data_ptr()
        args.q_workspace_bytes = ws.numel() * ws.element_size()


def paged_row_stats(q, dy, k_pool, v_pool, plan, *, causal=True, scale=None, out=None,
                    stream=None, split=True, workspace=None):
    """(max, denominator, delta) per (row, head) of the paged layout, float32
    [nq, heads, 3], computed on the GPU (attn_bwd_paged_row_stats).  split: use
    the split form (each block's tokens in pieces; a workspace is allocated
    unless one is given)."""
    torch = _torch()
    _io_dtype(q)
    nq, heads, D = q.shape
    if out is not None:  # checked as the call's input statistics below
        _check_float("out", out, torch.float32)
    if plan.device_words is None:
        plan.to(q.device)
    if out is None:
        out = torch.empty(nq, heads, 3, dtype=torch.float32, device=q.device)
    dummy = out  # the struct's input statistics are not read by this call
    args = make_paged_args(q, dy, k_pool, v_pool, dummy, plan, causal=causal, scale=scale)
    ws = None
    if split:
        ws = workspace if workspace is not None else paged_q_workspace(plan, D, q.device)
        _check_devices(q.device, [("workspace", ws)])
        _set_q_workspace(args, ws)
    handle, side = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_paged_row_stats(ctypes.byref(args), ctypes.c_void_p(out.data_ptr()),
                                                   handle))
    _record(side, out, ws, plan.device_words)
    return out


def attn_bwd_paged_dq(q, dy, k_pool, v_pool, stats, plan, *, causal=True, scale=None, out=None,
                      stream=None, split=True, workspace=None):
    """dQ [nq, heads, D] of the paged layout from the statistics (attn_bwd_paged_dq).
    split: as for paged_row_stats."""
    torch = _torch()
    dt = _io_dtype(q)
    if plan.device_words is None:
        plan.to(q.device)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args = make_paged_args(q, dy, k_pool, v_pool, stats, plan, causal=causal, scale=scale,
                           outs=[("dq", out, tuple(q.shape), dt)])
    ws = None
    if split:
        ws = workspace if workspace is not None else paged_q_workspace(plan, q.shape[2], q.device)
        _check_devices(q.device, [("workspace", ws)])
        _set_q_workspace(args, ws)
    handle, side = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_paged_dq(ctypes.byref(args), ctypes.c_void_p(out.data_ptr()),
                                            handle))
    _record(side, out, ws, plan.device_words)
    return out


def paged_stats_dq(q, dy, k_pool, v_pool, plan, *, causal=True, scale=None, stats_out=None,
                   dq_out=None, stream=None, form="auto", workspace=None):
    """The statistics [nq, heads, 3] and dQ [nq, heads, D] of the paged layout in
    one call (attn_bwd_paged_stats_dq: one pass over the tokens for bf16).
    form: "auto" (a workspace is allocated unless one is given, and the library
    picks the split or the direct form from the plan), "split" or "direct".
    Returns (stats, dq)."""
    torch = _torch()
    dt = _io_dtype(q)
    nq, heads, D = q.shape
    forms = {"auto": 0, "split": 1, "direct": 2}
    if form not in forms:
        raise ValueError(f"form must be one of {sorted(forms)}")
    if stats_out is not None:  # checked as the call's input statistics below
        _check_float("stats_out", stats_out, torch.float32)
    if plan.device_words is None:
        plan.to(q.device)
    if stats_out is None:
        stats_out = torch.empty(nq, heads, 3, dtype=torch.float32, device=q.device)
    if dq_out is None:
        dq_out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args = make_paged_args(q, dy, k_pool, v_pool, stats_out, plan, causal=causal, scale=scale,
                           outs=[("dq", dq_out, tuple(q.shape), dt)])
    args.q_form = forms[form]
    ws = None
    if form != "direct":
        ws = workspace if workspace is not None else paged_q_workspace(plan, D, q.device)
        _check_devices(q.device, [("workspace", ws)])
        _set_q_workspace(args, ws)
    handle, side = _launch_stream(stream, q.device)
    _check(load_library().attn_bwd_paged_stats_dq(ctypes.byref(args),
                                                  ctypes.c_void_p(stats_out.data_ptr()),
                                                  ctypes.c_void_p(dq_out.data_ptr()), handle))
    _record(side, stats_out, dq_out, ws, plan.device_words)
    return stats_out, dq_out
