"""Shared test helpers: building, input tensors, tolerance checks.

Inputs come from ``synth`` (seeded, shared with the oracle); expected values
come only from ``oracle``.  Nothing here computes attention or layouts.
"""
from __future__ import annotations

import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Parity bars: bf16 max |err| <= 2e-2 and rel. RMS <= 1e-2; fp32 both <= 1e-4.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
# bf16 unit roundoff (8 significant bits, round to nearest even).
BF16_U = 2.0 ** -8


def ensure_library():
    """Load libulysses, building it only when no build exists."""
    import ulysses_sp_attention_amd as uly
    if not os.path.exists(uly.LIB_PATH):
        from ulysses_sp_attention_amd import _build
        _build.build_lib()
    return uly.load_library()


def to_device(arr: np.ndarray, dtype: str):
    """Host storage (bf16 bits as uint16, or f32) -> device tensor of that dtype."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def to_f64(t) -> np.ndarray:
    """Exact float64 value of a device tensor (bf16 or f32)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def storage_bytes(t) -> bytes:
    """Raw bytes of a tensor's storage (for bit-exact comparisons)."""
    import torch
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        c = c.view(torch.int16)
    return c.numpy().tobytes()


def host_storage(t) -> np.ndarray:
    """Device tensor -> host array in generator storage form (uint16 bits or f32)."""
    import torch
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def errors(got: np.ndarray, want: np.ndarray):
    """(max abs error, relative RMS error) of got against want."""
    d = np.asarray(got, np.float64) - np.asarray(want, np.float64)
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    denom = float(np.sqrt(np.sum(np.square(want)))) or 1.0
    return max_abs, float(np.sqrt(np.sum(np.square(d)))) / denom


def assert_close(got, want, dtype: str, what: str = "", mag=None, k_u: float = 2.0, d_mag=None):
    """Parity bar.  Relative RMS error <= the dtype's bar, and elementwise

        |err| <= max(tol_abs, u * (k_u * mag + d_mag))   for bf16 results given mag,
        |err| <= tol_abs                                 otherwise,

    with u = 2^-8 (bf16 unit roundoff) and ``mag`` the oracle's sum of
    |terms| behind each output.  A sum whose operands carry r bf16 roundings
    and whose result is rounded once to bf16 is off by at most (r + 1) u mag
    (first order), so k_u = r + 1 is the count of roundings on the path:
    2 for O (P rounded), dV (P rounded) and dQ (dS rounded), 3 for dK (dS
    formed from the rounded P and rounded again).  Where that bound is below
    tol_abs the stated bar applies unchanged; it is only wider for outputs
    whose magnitude puts tol_abs below bf16's own resolution.  ``d_mag``
    (gradients after a bf16 forward only) is the oracle's sensitivity of the
    output to D = <dO, O>: the backward sees O rounded once to bf16, which
    moves D by at most u sum_e |dO_e| (P|V|)_e and the output by at most
    u * d_mag."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    max_abs, rel = errors(got, want)
    tol_abs, tol_rel = TOL[dtype]
    bound = np.full(want.shape, tol_abs)
    if mag is not None and dtype == "bf16":
        extra = 0.0 if d_mag is None else np.asarray(d_mag, np.float64)
        bound = np.maximum(bound, BF16_U * (k_u * np.asarray(mag, np.float64) + extra))
    excess = np.abs(got - want) - bound
    worst = int(np.argmax(excess)) if excess.size else 0
    ok = (excess.size == 0 or excess.flat[worst] <= 0) and rel <= tol_rel
    assert ok, (f"{what}: rel_rms={rel:.3e} (tol {tol_rel}); max_abs={max_abs:.3e}; worst element "
                f"{np.unravel_index(worst, want.shape)} err={abs(got.flat[worst] - want.flat[worst]):.3e}"
                f" bound={bound.flat[worst]:.3e} ref={want.flat[worst]:.4f}")
    return max_abs, rel


def assert_rows_close(got, want, dtype: str, what: str = ""):
    """Per-row relative bar: for every row of the last axis (one head of one
    position), ||err||_2 <= tol_rel * ||ref||_2, with tol_rel the dtype's
    relative bar.  This sees a wrong row whose elements all lie below the
    elementwise absolute bar (e.g. late rows of a long causal share, whose
    outputs average tens of thousands of values).  It applies to outputs
    that are probability-weighted sums with no cancellation built in (O and
    dV), whose bf16 error stays a small fraction of every row.  dQ and dK are
    not held to it: their terms dS_ij sum to exactly zero over a row of
    keys, so a row can be small against the sum of its |terms|, and there
    the bf16 rounding of dS and D bounds the error absolutely (the
    elementwise bar with the oracle's magnitudes), not relative to the row.
    Rows whose reference norm is zero or below 1e-3 of the median row norm
    are left to the elementwise bar."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol_rel = TOL[dtype][1]
    hd = want.shape[-1]
    d = np.sqrt(np.sum(np.square((got - want).reshape(-1, hd)), axis=1))
    r = np.sqrt(np.sum(np.square(want.reshape(-1, hd)), axis=1))
    if r.size == 0:
        return 0.0
    live = (r > 0) & (r >= 1e-3 * np.median(r))
    ratio = np.where(live, d / np.where(live, r, 1.0), 0.0)
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= tol_rel, (
        f"{what}: row {np.unravel_index(worst, want.shape[:-1])} relative error {ratio[worst]:.3e} "
        f"(tol {tol_rel}), |ref| = {r[worst]:.3e}")
    return float(ratio[worst])


def assert_grads_close(dtype: str, dq, dk, dv, ref, what: str = "fwd+bwd"):
    """Gradients (float64 arrays) of a GPU forward then backward against the
    exact gradient ``ref`` = oracle.attn_bwd(..., magnitude=True).  Besides
    its own roundings, the backward sees O rounded to the storage format, so
    D_i is off by up to u sum_e |dO_ie| (P|V|)_ie; the oracle's
    dq_from_D/dk_from_D carry that through to dQ and dK.  Every key row of
    dV is also held to the per-row relative bar (see assert_rows_close)."""
    dq_ref, dk_ref, dv_ref, m = ref
    assert_close(dq, dq_ref, dtype, f"dQ ({what})", m["dq"], d_mag=m["dq_from_D"])
    assert_close(dk, dk_ref, dtype, f"dK ({what})", m["dk"], k_u=3, d_mag=m["dk_from_D"])
    assert_close(dv, dv_ref, dtype, f"dV ({what})", m["dv"])
    assert_rows_close(dv, dv_ref, dtype, f"dV rows ({what})")


def sample_rows(N: int, seed: int, n_first=256, n_last=256, n_rand=1024) -> np.ndarray:
    """First and last rows plus seeded random ones (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(n_first, N))) | set(range(max(0, N - n_last), N))
    rows |= set(int(x) for x in rng.integers(0, N, size=n_rand))
    return np.array(sorted(rows), dtype=np.int64)


def head_inputs(w: synth.Workload, streams=(synth.STREAM_Q, synth.STREAM_K, synth.STREAM_V)):
    """Head-sharded host inputs generated directly ([N, bs, heads_l, hd])."""
    out = []
    for s in streams:
        heads = w.hkv_local if s in (synth.STREAM_K, synth.STREAM_V) else w.hq_local
        scale = w.q_prescale if s == synth.STREAM_Q else 1.0
        out.append(w.head_tensor(s, heads, scale=scale))
    return out
