"""CPU float64 oracle for scaled dot-product attention backward.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the benchmark's ``cpu_baseline`` leg, never by the GPU product path.
It shares no code with the HIP library (``scaled_dot_product_bwd_amd``) and does
not import it.

The arithmetic lives in ``attn_oracle.c`` (plain C, float64, one thread per
(batch, head) head).  This module only marshals arrays: it converts inputs to
contiguous float64 ``[B, S, H, D]`` numpy arrays, calls the C functions through
ctypes and returns numpy arrays.

Sources, cited by page title and function:
  rlx-cpu 0.2.17 src/attention_bwd.rs (`backward_dense_head_all`,
  `apply_synthetic_mask`), rlx-wgpu 0.2.1 src/kernels/attention_bwd.wgsl
  (`mask_score`, `softmax_row`), ruDNN 0.1.43
  src/paged_attention/ordered_kernel.rs (`history_backward`).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build as _build, library_path

MASK_NONE, MASK_CAUSAL, MASK_KEYPAD, MASK_WINDOW, MASK_BIAS = 0, 1, 2, 3, 4

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        _build()
    lib = ctypes.CDLL(path)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp,
                                    i32, i32, i64, _dp, _lp, dbl, dbl,
                                    _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, i32]
    paged = [i32, _ip, _ip, i32, i32, _ip, _ip, i32, i32, i32, i32, i32, i32, dbl,
             _dp, _dp, _dp, _dp]
    lib.oracle_paged_row_stats.restype = ctypes.c_int
    lib.oracle_paged_row_stats.argtypes = paged + [_dp, ctypes.c_int]
    lib.oracle_paged_kv_bwd.restype = ctypes.c_int
    lib.oracle_paged_kv_bwd.argtypes = paged + [_dp, _dp, _dp, ctypes.c_int]
    lib.oracle_paged_dq.restype = ctypes.c_int
    lib.oracle_paged_dq.argtypes = paged + [_dp, _dp, ctypes.c_int]
    mla = [i32, _ip, _ip, i32, i32, _ip, _ip, i32, i32, i32, i32, i32, i32, i32, dbl,
           _dp, _dp, _dp, _dp, _dp]
    lib.oracle_paged_mla_row_stats.restype = ctypes.c_int
    lib.oracle_paged_mla_row_stats.argtypes = mla + [_dp, ctypes.c_int]
    lib.oracle_paged_mla_kv_bwd.restype = ctypes.c_int
    lib.oracle_paged_mla_kv_bwd.argtypes = mla + [_dp, _dp, _dp, ctypes.c_int]
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Any array-like (numpy, torch CPU tensor of any float dtype) -> contiguous float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


def attn_bwd(q, k, v, dy, *, mask_kind=MASK_NONE, causal_flag=False, window=0,
             mask=None, threshold=0.5, scale=None, nthreads=None):
    """Dense backward for ``[B, S, H, D]`` inputs.

    ``mask`` (keypad validity or additive bias) is any array that broadcasts to
    ``[B, H, Sq, Sk]``; broadcast axes are passed as zero strides.
    ``scale`` defaults to the float32 value of 1/sqrt(D), promoted to float64,
    as rlx-cpu `backward_dense_head_all` computes it in f32.

    Returns a dict of float64 arrays: dq, dk, dv ([B, S, H, D]); m, l, delta,
    delta_o ([B, H, Sq]); out (forward output O, [B, Sq, H, D]).
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    assert k.shape == (B, Sk, H, D) and v.shape == k.shape and dy.shape == q.shape
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    mview, mst = None, None
    if mask_kind in (MASK_KEYPAD, MASK_BIAS):
        m64 = _f64(mask)
        mview = np.broadcast_to(m64, (B, H, Sq, Sk))
        mst = np.array([s // 8 for s in mview.strides], dtype=np.int64)
    res = {
        "dq": np.empty((B, Sq, H, D)), "dk": np.empty((B, Sk, H, D)),
        "dv": np.empty((B, Sk, H, D)), "m": np.empty((B, H, Sq)),
        "l": np.empty((B, H, Sq)), "delta": np.empty((B, H, Sq)),
        "delta_o": np.empty((B, H, Sq)), "out": np.empty((B, Sq, H, D)),
    }
    lib = _load()
    rc = lib.oracle_attn_bwd(
        B, H, Sq, Sk, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dy),
        int(mask_kind), int(bool(causal_flag)), int(window),
        None if mview is None else ctypes.cast(mview.ctypes.data, _dp),
        None if mst is None else mst.ctypes.data_as(_lp),
        float(threshold), float(scale),
        _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["m"]),
        _ptr(res["l"]), _ptr(res["delta"]), _ptr(res["delta_o"]), _ptr(res["out"]),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd rejected its arguments (rc={rc})")
    return res


def attn_bwd_gqa(q, k, v, dy, **kw):
    """Grouped-query backward: K, V ``[B, Sk, Hkv, D]`` serve ``H / Hkv`` query
    heads each (query head h reads KV head h // (H / Hkv)).  By definition the
    forward equals the dense one with each KV head repeated over its group, so
    dQ is that problem's dQ and dK, dV are its dK, dV summed over each group.
    Same keywords and result keys as `attn_bwd` (dk, dv with Hkv heads)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, Hkv = q.shape[2], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    g = H // Hkv
    res = attn_bwd(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), dy, **kw)
    B, Sk, _, D = k.shape
    res["dk"] = res["dk"].reshape(B, Sk, Hkv, g, D).sum(axis=3)
    res["dv"] = res["dv"].reshape(B, Sk, Hkv, g, D).sum(axis=3)
    return res


def _paged_common(w):
    seq_lens = _i32(w["seq_lens"])
    bt = _i32(w["block_table"])
    nseq, max_pages = bt.shape
    qs, qp = _i32(w["query_seq"]), _i32(w["query_pos"])
    return seq_lens, bt, nseq, max_pages, qs, qp


def paged_row_stats(w, q, dy, k_pool, v_pool, *, heads, kv_heads, page_size,
                    causal=True, scale=None, nthreads=None):
    """(max, denominator, delta) per (row, head) for the paged layout, shape [nq, heads, 3]."""
    seq_lens, bt, nseq, max_pages, qs, qp = _paged_common(w)
    q, dy, kp, vp = _f64(q), _f64(dy), _f64(k_pool), _f64(v_pool)
    nq, _, D = q.shape
    pool_pages = kp.shape[0] // page_size
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    stats = np.empty((nq, heads, 3))
    rc = _load().oracle_paged_row_stats(
        nseq, _ptr(seq_lens, _ip), _ptr(bt, _ip), max_pages, nq, _ptr(qs, _ip),
        _ptr(qp, _ip), heads, kv_heads, D, page_size, pool_pages, int(bool(causal)),
        float(scale), _ptr(q), _ptr(dy), _ptr(kp), _ptr(vp), _ptr(stats),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_row_stats rejected its arguments (rc={rc})")
    return stats


def paged_kv_bwd(w, q, dy, k_pool, v_pool, stats, dk_init, dv_init, *, heads,
                 kv_heads, page_size, causal=True, scale=None, nthreads=None):
    """dK, dV pools: listed pages' slots overwritten, all other slots = the *_init contents."""
    seq_lens, bt, nseq, max_pages, qs, qp = _paged_common(w)
    q, dy, kp, vp, st = _f64(q), _f64(dy), _f64(k_pool), _f64(v_pool), _f64(stats)
    dk, dv = _f64(dk_init).copy(), _f64(dv_init).copy()
    nq, _, D = q.shape
    pool_pages = kp.shape[0] // page_size
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    rc = _load().oracle_paged_kv_bwd(
        nseq, _ptr(seq_lens, _ip), _ptr(bt, _ip), max_pages, nq, _ptr(qs, _ip),
        _ptr(qp, _ip), heads, kv_heads, D, page_size, pool_pages, int(bool(causal)),
        float(scale), _ptr(q), _ptr(dy), _ptr(kp), _ptr(vp), _ptr(st), _ptr(dk), _ptr(dv),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_kv_bwd rejected its arguments (rc={rc})")
    return dk, dv


def paged_dq(w, q, dy, k_pool, v_pool, stats, *, heads, kv_heads, page_size, causal=True,
             scale=None, nthreads=None):
    """dQ [nq, heads, D] of the paged layout from the given (max, denominator, delta)."""
    seq_lens, bt, nseq, max_pages, qs, qp = _paged_common(w)
    q, dy, kp, vp, st = _f64(q), _f64(dy), _f64(k_pool), _f64(v_pool), _f64(stats)
    nq, _, D = q.shape
    pool_pages = kp.shape[0] // page_size
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    dq = np.empty((nq, heads, D))
    rc = _load().oracle_paged_dq(
        nseq, _ptr(seq_lens, _ip), _ptr(bt, _ip), max_pages, nq, _ptr(qs, _ip),
        _ptr(qp, _ip), heads, kv_heads, D, page_size, pool_pages, int(bool(causal)),
        float(scale), _ptr(q), _ptr(dy), _ptr(kp), _ptr(vp), _ptr(st), _ptr(dq),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_dq rejected its arguments (rc={rc})")
    return dq


def _mla_scale(D, P, scale):
    # the score contracts over the latent and the position parts together
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D + P)))
    return float(scale)


def paged_mla_row_stats(w, q, qp, dy, latent_pool, kp_pool, *, heads, kv_heads, page_size,
                        causal=True, scale=None, nthreads=None):
    """Latent variant: (max, denominator, delta) per (row, head), shape [nq, heads, 3].

    q, dy: [nq, heads, D] (latent width); qp: [nq, heads, P]; latent_pool:
    [slots, kv_heads, D] (both key and value); kp_pool: [slots, kv_heads, P].
    The default scale is 1/sqrt(D + P) (the score's contraction width)."""
    seq_lens, bt, nseq, max_pages, qs, qpos = _paged_common(w)
    q, qp, dy = _f64(q), _f64(qp), _f64(dy)
    lat, kp = _f64(latent_pool), _f64(kp_pool)
    nq, _, D = q.shape
    P = qp.shape[2]
    pool_pages = lat.shape[0] // page_size
    stats = np.empty((nq, heads, 3))
    rc = _load().oracle_paged_mla_row_stats(
        nseq, _ptr(seq_lens, _ip), _ptr(bt, _ip), max_pages, nq, _ptr(qs, _ip),
        _ptr(qpos, _ip), heads, kv_heads, D, P, page_size, pool_pages, int(bool(causal)),
        _mla_scale(D, P, scale), _ptr(q), _ptr(qp), _ptr(dy), _ptr(lat), _ptr(kp), _ptr(stats),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_mla_row_stats rejected its arguments (rc={rc})")
    return stats


def paged_mla_kv_bwd(w, q, qp, dy, latent_pool, kp_pool, stats, dlat_init, dkp_init, *,
                     heads, kv_heads, page_size, causal=True, scale=None, nthreads=None):
    """Latent variant: (d latent, d position key) pools; listed pages' slots
    overwritten, all other slots = the *_init contents."""
    seq_lens, bt, nseq, max_pages, qs, qpos = _paged_common(w)
    q, qp, dy, st = _f64(q), _f64(qp), _f64(dy), _f64(stats)
    lat, kp = _f64(latent_pool), _f64(kp_pool)
    dlat, dkp = _f64(dlat_init).copy(), _f64(dkp_init).copy()
    nq, _, D = q.shape
    P = qp.shape[2]
    pool_pages = lat.shape[0] // page_size
    rc = _load().oracle_paged_mla_kv_bwd(
        nseq, _ptr(seq_lens, _ip), _ptr(bt, _ip), max_pages, nq, _ptr(qs, _ip),
        _ptr(qpos, _ip), heads, kv_heads, D, P, page_size, pool_pages, int(bool(causal)),
        _mla_scale(D, P, scale), _ptr(q), _ptr(qp), _ptr(dy), _ptr(lat), _ptr(kp), _ptr(st),
        _ptr(dlat), _ptr(dkp), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_paged_mla_kv_bwd rejected its arguments (rc={rc})")
    return dlat, dkp


__all__ = ["attn_bwd", "attn_bwd_gqa", "paged_row_stats", "paged_kv_bwd", "paged_dq",
           "paged_mla_row_stats", "paged_mla_kv_bwd", "MASK_NONE", "MASK_CAUSAL",
           "MASK_KEYPAD", "MASK_WINDOW", "MASK_BIAS", "default_threads"]
