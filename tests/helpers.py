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


def assert_close(got, want, dtype: str, what: str = "", mag=None):
    """Parity bar.  Relative RMS error <= the dtype's bar.  Elementwise
    |err| <= the dtype's absolute bar, widened for bf16 results by the
    rounding error bound of the arithmetic when ``mag`` -- the oracle's sum of
    |terms| behind each output -- is given: a bf16 sum whose operands and
    result are each rounded once can be off by 2 * u * mag, u = 2^-8, which
    exceeds 2e-2 as soon as mag > 2.56 (e.g. gradients of magnitude 10-30)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    max_abs, rel = errors(got, want)
    tol_abs, tol_rel = TOL[dtype]
    bound = np.full(want.shape, tol_abs)
    if mag is not None and dtype == "bf16":
        bound = bound + 2.0 * BF16_U * np.asarray(mag, np.float64)
    excess = np.abs(got - want) - bound
    worst = int(np.argmax(excess)) if excess.size else 0
    ok = (excess.size == 0 or excess.flat[worst] <= 0) and rel <= tol_rel
    assert ok, (f"{what}: rel_rms={rel:.3e} (tol {tol_rel}); max_abs={max_abs:.3e}; worst element "
                f"{np.unravel_index(worst, want.shape)} err={abs(got.flat[worst] - want.flat[worst]):.3e}"
                f" bound={bound.flat[worst]:.3e} ref={want.flat[worst]:.4f}")
    return max_abs, rel


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
