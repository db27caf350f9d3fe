"""The backward entry point that allocates nothing (ulysses_attn_bwd_noalloc),
through the C-ABI, against the workspace entry point (ulysses_attn_bwd) it
varies: the same kernels with the statistics (and, where they fit, the dK/dV
split's partials) in the library's fixed per-GPU scratch instead of a
caller's workspace.  Where the split's partials fit the scratch both run the
same launches and must agree bit for bit (which is within every parity
bar): two calls in a row on the shared scratch, the second smaller, each
checked; then the first again, to show that the contents a smaller call
leaves behind do not matter.  Where they do not fit, the scratch entry point
runs dK/dV unsplit, which changes the order of one fp32 sum: both results are
then held to the parity bar against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_grads_close, ensure_library, storage_bytes, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def case_inputs(N, hq, hkv, hd, dtype, seed):
    q = to_device(synth.normal(seed, synth.STREAM_Q, (N, 1, hq, hd), dtype, scale=0.5), dtype)
    k = to_device(synth.normal(seed, synth.STREAM_K, (N, 1, hkv, hd), dtype), dtype)
    v = to_device(synth.normal(seed, synth.STREAM_V, (N, 1, hkv, hd), dtype), dtype)
    do = to_device(synth.normal(seed, synth.STREAM_DO, (N, 1, hq, hd), dtype), dtype)
    return q, k, v, do


def run_both(N, hq, hkv, hd, dtype, cu, seed):
    """(inputs, workspace-entry-point gradients, scratch-entry-point gradients)."""
    import torch
    import ulysses_sp_attention_amd as uly
    q, k, v, do = case_inputs(N, hq, hkv, hd, dtype, seed)
    scale = 1.0 / np.sqrt(hd)
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((1, hq, N), dtype=torch.float32, device="cuda")
    uly.ulysses_attn_fwd(q, k, v, o, lse, scale, True, cu_t)
    code = uly.BF16 if dtype == "bf16" else uly.FP32
    ws = torch.full((uly.ulysses_attn_bwd_workspace_size(N, 1, hq, hkv, hd, code) // 4,),
                    float("nan"), dtype=torch.float32, device="cuda")
    want = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    uly.ulysses_attn_bwd(q, k, v, o, lse, do, *want, ws, scale, True, cu_t)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    uly.ulysses_attn_bwd_noalloc(q, k, v, o, lse, do, *got, scale, True, cu_t)
    torch.cuda.synchronize()
    for name, g in zip(("dq", "dk", "dv"), got):
        assert not torch.isnan(g.float()).any(), name
    return (q, k, v, do, scale), want, got


def run_case(N, hq, hkv, hd, dtype, cu, seed):
    _, want, got = run_both(N, hq, hkv, hd, dtype, cu, seed)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert storage_bytes(g) == storage_bytes(w), f"{name} differs at N={N}"


CASES = [
    # N, hq, hkv, hd, dtype, cu: the 32K share's head counts at 2K rows (the
    # dK/dV split's partials, 8 MiB, fit the scratch), then smaller
    (2048, 4, 1, 128, "bf16", None),
    (777, 8, 2, 64, "bf16", [0, 100, 101, 777]),
]


def test_noalloc_backward_equals_workspace_backward_two_calls():
    for i, (N, hq, hkv, hd, dtype, cu) in enumerate(CASES):
        run_case(N, hq, hkv, hd, dtype, cu, seed=900 + i)
    # the large case again, after the smaller one left its statistics behind
    N, hq, hkv, hd, dtype, cu = CASES[0]
    run_case(N, hq, hkv, hd, dtype, cu, seed=900)


def test_noalloc_backward_unsplit_when_partials_do_not_fit():
    """At 4160 rows of 4 heads the split's fp32 partials (17 MB) exceed the
    16 MiB scratch: the scratch entry point runs dK/dV unsplit and the two
    entry points' dK/dV may differ in the last bit; dQ (no split) agrees bit
    for bit, and both sets of gradients meet the parity bar against the
    oracle, end to end from the same GPU forward."""
    N, hq, hkv, hd = 4160, 4, 1, 128
    (q, k, v, do, scale), want, got = run_both(N, hq, hkv, hd, "bf16", None, seed=907)
    assert storage_bytes(got[0]) == storage_bytes(want[0])
    ref = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, True, None,
                          magnitude=True)
    for what, grads in (("workspace entry point", want), ("scratch entry point", got)):
        assert_grads_close("bf16", *(to_f64(t) for t in grads), ref, what)


def test_noalloc_backward_fp32():
    run_case(300, 4, 2, 64, "f32", None, seed=905)
    run_case(97, 2, 1, 32, "f32", [0, 50, 97], seed=906)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """bf16 needs 8 bytes of statistics per (position, head): 2^21 rows fill
    the 16 MiB scratch; one more 64-position block is refused before any HIP
    call (the fake pointers are never dereferenced)."""
    import ulysses_sp_attention_amd as uly
    lib = uly.load_library()
    fake = 0x10000
    N = uly.NOALLOC_SCRATCH_BYTES // 8 // 4 + 64   # 4 heads
    st = lib.ulysses_attn_bwd_noalloc(fake, fake, fake, fake, fake, fake, N, 1, 4, 1, 128,
                                      uly.BF16, 0.088, 1, None, 0, fake, fake, fake, None)
    assert st == uly.ERR_WORKSPACE
