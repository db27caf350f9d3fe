"""ORACLE -- test infrastructure only.

Python access to the plain fp64 CPU statement of one rank's share of an
Ulysses attention layer (``oracle.c``).  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import this package; the product path
(``ulysses_sp_attention_amd``) never does, and the two share no code.

Every function takes and returns numpy arrays:

* permutations work on raw storage (any dtype) and are bit copies;
* attention takes float64 arrays [N, bs, heads, hd] holding the exact input
  values and returns float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point this at a deliberately broken build of oracle.c to show
# that the pins catch the mistake (tests/test_oracle_mutants.py); that build
# is never made here.
_LIB_OVERRIDE = os.environ.get("ULYSSES_ORACLE_LIB")
_lib = None


def build_lib() -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, ci, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ci
    lib.oracle_attn_merge.argtypes = [vp, vp, vp, vp, i64, ci, ci, ci, vp, vp]
    lib.oracle_logits_loss.argtypes = [vp, vp, vp, i64, i64, i64, i64, dbl, vp, vp, vp, vp, vp, vp,
                                       vp, vp]
    lib.oracle_logits_loss.restype = ci
    lib.oracle_swiglu_mlp.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64] + [vp] * 10
    lib.oracle_swiglu_mlp.restype = ci
    lib.oracle_attn_merge.restype = ci
    lib.oracle_seq_to_head.argtypes = [vp, ci, ci, i64, ci, ci, ci, ci, vp]
    lib.oracle_seq_to_head.restype = ci
    lib.oracle_head_to_seq.argtypes = [vp, ci, ci, i64, ci, ci, ci, ci, vp]
    lib.oracle_head_to_seq.restype = ci
    lib.oracle_attn_fwd.argtypes = [vp, vp, vp, i64, ci, ci, ci, ci, dbl, ci, vp, ci, vp, i64, vp, vp, vp]
    lib.oracle_attn_fwd.restype = ci
    lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i64, ci, ci, ci, ci, dbl, ci, vp, ci,
                                    vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_attn_bwd.restype = ci
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data
    return arr


def _local_heads(heads: int, P: int) -> int:
    return heads // P if heads >= P else 1


def seq_to_head(chunks, rank: int) -> np.ndarray:
    """P seq-sharded chunks [n, bs, heads, hd] -> rank's [P*n, bs, heads_l, hd]."""
    P = len(chunks)
    n, bs, heads, hd = chunks[0].shape
    for c in chunks:
        if c.shape != chunks[0].shape or c.dtype != chunks[0].dtype or not c.flags.c_contiguous:
            raise ValueError("chunks must be contiguous and alike")
    out = np.empty((P * n, bs, _local_heads(heads, P), hd), dtype=chunks[0].dtype)
    rc = _load().oracle_seq_to_head(_ptr_array(chunks), P, rank, n, bs, heads, hd,
                                    chunks[0].itemsize, out.ctypes.data)
    if rc:
        raise ValueError("oracle_seq_to_head: bad arguments")
    return out


def head_to_seq(x: np.ndarray, chunks, rank: int) -> None:
    """Rank's [P*n, bs, heads_l, hd] -> its head slots of the P chunks (in place)."""
    P = len(chunks)
    n, bs, heads, hd = chunks[0].shape
    if x.shape != (P * n, bs, heads // P, hd) or not x.flags.c_contiguous:
        raise ValueError("bad head-sharded input shape")
    rc = _load().oracle_head_to_seq(x.ctypes.data, P, rank, n, bs, heads, hd, x.itemsize,
                                    _ptr_array(chunks))
    if rc:
        raise ValueError("oracle_head_to_seq: bad arguments")


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _cu64(cu):
    return None if cu is None else np.ascontiguousarray(cu, dtype=np.int64)


def attn_fwd(q, k, v, scale: float, causal: bool = True, cu_seqlens=None, rows=None,
             magnitude: bool = False):
    """Returns (O, LSE): O [nsel, bs, hq, hd], LSE [bs, hq, nsel] (nsel = N or len(rows)).
    With magnitude=True returns (O, LSE, M) where M = sum_j P_ij |v_j| (O's layout)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, bs, hq, hd = q.shape
    hkv = k.shape[2]
    cu = _cu64(cu_seqlens)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nsel = N if rows_a is None else len(rows_a)
    o = np.empty((nsel, bs, hq, hd))
    lse = np.empty((bs, hq, nsel))
    mag = np.empty_like(o) if magnitude else None
    rc = _load().oracle_attn_fwd(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, N, bs, hq, hkv, hd, float(scale), int(causal),
        None if cu is None else cu.ctypes.data, 0 if cu is None else len(cu) - 1,
        None if rows_a is None else rows_a.ctypes.data, nsel, o.ctypes.data, lse.ctypes.data,
        None if mag is None else mag.ctypes.data)
    if rc:
        raise ValueError("oracle_attn_fwd: bad arguments")
    return (o, lse, mag) if magnitude else (o, lse)


def attn_bwd(q, k, v, dout, scale: float, causal: bool = True, cu_seqlens=None,
             dq_rows=None, dkv_cols=None, magnitude: bool = False, o=None, lse=None):
    """Returns (dQ, dK, dV), compact over the selected rows / columns.

    o, lse: optional forward outputs to use in place of the oracle's own (full
    [N, bs, hq, hd] and [bs, hq, N]), as a backward call receives them.
    With magnitude=True returns (dQ, dK, dV, mags) where mags is a dict:
    "dq", "dk", "dv" -- each output sum re-evaluated with every term replaced
    by its absolute value; "dq_from_D", "dk_from_D" -- the sensitivity of dQ
    and dK to the magnitude of D (see oracle.c)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    o_in = None if o is None else _f64(o)
    lse_in = None if lse is None else _f64(lse)
    N, bs, hq, hd = q.shape
    hkv = k.shape[2]
    cu = _cu64(cu_seqlens)
    qr = None if dq_rows is None else np.ascontiguousarray(dq_rows, dtype=np.int64)
    kc = None if dkv_cols is None else np.ascontiguousarray(dkv_cols, dtype=np.int64)
    nq = N if qr is None else len(qr)
    nk = N if kc is None else len(kc)
    dq = np.empty((nq, bs, hq, hd))
    dk = np.empty((nk, bs, hkv, hd))
    dv = np.empty((nk, bs, hkv, hd))
    mags = ((np.empty_like(dq), np.empty_like(dk), np.empty_like(dv), np.empty_like(dq),
             np.empty_like(dk)) if magnitude else (None,) * 5)
    # a zero-length selection still needs a valid (non-NULL) pointer
    dummy = np.zeros(1, np.int64)
    qr_p = None if qr is None else (qr if nq else dummy).ctypes.data
    kc_p = None if kc is None else (kc if nk else dummy).ctypes.data
    rc = _load().oracle_attn_bwd(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, N, bs, hq, hkv, hd,
        float(scale), int(causal), None if cu is None else cu.ctypes.data,
        0 if cu is None else len(cu) - 1, qr_p, nq, kc_p, nk,
        None if o_in is None else o_in.ctypes.data, None if lse_in is None else lse_in.ctypes.data,
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
        *[None if m is None else m.ctypes.data for m in mags])
    if rc:
        raise ValueError("oracle_attn_bwd: bad arguments")
    if not magnitude:
        return dq, dk, dv
    return dq, dk, dv, dict(zip(("dq", "dk", "dv", "dq_from_D", "dk_from_D"), mags))


def attn_merge(o_a, lse_a, o_b, lse_b):
    """Merge of two partial attention results over disjoint key sets (see
    oracle.c): returns (O, LSE) with O [N, bs, heads, hd] and LSE [bs, heads, N]."""
    o_a, o_b, lse_a, lse_b = _f64(o_a), _f64(o_b), _f64(lse_a), _f64(lse_b)
    N, bs, heads, hd = o_a.shape
    if o_b.shape != o_a.shape or lse_a.shape != (bs, heads, N) or lse_b.shape != (bs, heads, N):
        raise ValueError("attn_merge: shape mismatch")
    o = np.empty_like(o_a)
    lse = np.empty_like(lse_a)
    rc = _load().oracle_attn_merge(o_a.ctypes.data, lse_a.ctypes.data, o_b.ctypes.data,
                                   lse_b.ctypes.data, N, bs, heads, hd, o.ctypes.data,
                                   lse.ctypes.data)
    if rc:
        raise ValueError("oracle_attn_merge: bad arguments")
    return o, lse


IGNORE_INDEX = -100


def logits_loss(h, w, labels, grad_scale: float = 1.0, ignore_index: int = IGNORE_INDEX,
                magnitude: bool = False):
    """Cross-entropy of the lm_head logits h W^T against (already shifted)
    labels and its gradients (see oracle.c).  h [T, d], w [V, d], labels [T].
    Returns (loss_rows [T], loss_sum, n_good, dh [T, d], dw [V, d]); with
    magnitude=True also a dict of rounding-bound magnitudes (zmag [T],
    dh [T, d], dw [V, d])."""
    h, w = _f64(h), _f64(w)
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    T, d = h.shape
    V = w.shape[0]
    if w.shape != (V, d) or labels.shape != (T,):
        raise ValueError("logits_loss: shape mismatch")
    loss_rows = np.empty(T)
    loss_sum = np.empty(1)
    n_good = np.empty(1, dtype=np.int64)
    dh = np.empty((T, d))
    dw = np.empty((V, d))
    mags = [np.empty(T), np.empty((T, d)), np.empty((V, d))] if magnitude else [None] * 3
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _load().oracle_logits_loss(ptr(h), ptr(w), ptr(labels), T, d, V, ignore_index,
                                    grad_scale, ptr(loss_rows), ptr(loss_sum), ptr(n_good),
                                    ptr(dh), ptr(dw), *[ptr(m) for m in mags])
    if rc:
        raise ValueError(f"oracle_logits_loss: bad arguments ({rc})")
    out = (loss_rows, float(loss_sum[0]), int(n_good[0]), dh, dw)
    if magnitude:
        return out + (dict(zip(("zmag", "dh", "dw"), mags)),)
    return out


def swiglu_mlp(x, wg, wu, wd, dy=None, magnitude: bool = False):
    """SwiGLU MLP y = (silu(x Wg^T) * (x Wu^T)) Wd^T and, with dy, its
    gradients (see oracle.c).  x [T, d], wg and wu [I, d], wd [d, I].
    Returns y, or (y, dx, dwg, dwu, dwd) with dy; with magnitude=True a dict
    of rounding-bound magnitudes is appended."""
    x, wg, wu, wd = _f64(x), _f64(wg), _f64(wu), _f64(wd)
    T, d = x.shape
    I = wg.shape[0]
    if wg.shape != (I, d) or wu.shape != (I, d) or wd.shape != (d, I):
        raise ValueError("swiglu_mlp: shape mismatch")
    bwd = dy is not None
    if bwd:
        dy = _f64(dy)
        if dy.shape != (T, d):
            raise ValueError("swiglu_mlp: dy shape")
    y = np.empty((T, d))
    grads = [np.empty((T, d)), np.empty((I, d)), np.empty((I, d)), np.empty((d, I))] if bwd \
        else [None] * 4
    names = ("y", "dx", "dwg", "dwu", "dwd")
    shapes = ((T, d), (T, d), (I, d), (I, d), (d, I))
    mags = [np.empty(sh) if magnitude and (bwd or n == "y") else None
            for n, sh in zip(names, shapes)]
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = _load().oracle_swiglu_mlp(ptr(x), ptr(wg), ptr(wu), ptr(wd), ptr(dy), T, d, I, ptr(y),
                                   *[ptr(g) for g in grads], *[ptr(m) for m in mags])
    if rc:
        raise ValueError(f"oracle_swiglu_mlp: bad arguments ({rc})")
    out = (y,) + (tuple(grads) if bwd else ())
    if magnitude:
        out = out + ({n: m for n, m in zip(names, mags) if m is not None},)
    return out if (bwd or magnitude) else y
