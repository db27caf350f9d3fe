"""The backward entry point that allocates nothing (ulysses_attn_bwd_noalloc),
through the C-ABI, against the workspace entry point (ulysses_attn_bwd) it
varies: the same kernels with the statistics in the library's fixed per-GPU
scratch instead of a caller's workspace, so the gradients must agree bit for
bit (which is within every parity bar).  Two calls in a row on the shared
scratch, the second smaller, each checked; then the first again, to show
that the contents a smaller call leaves behind do not matter."""
import numpy as np
import pytest

import synth
from helpers import ensure_library, storage_bytes, to_device

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


def run_case(N, hq, hkv, hd, dtype, cu, seed):
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
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert storage_bytes(g) == storage_bytes(w), f"{name} differs at N={N}"
        assert not torch.isnan(g.float()).any(), name


CASES = [
    # N, hq, hkv, hd, dtype, cu: the 32K share's head counts at 16K rows, then smaller
    (16384, 4, 1, 128, "bf16", None),
    (777, 8, 2, 64, "bf16", [0, 100, 101, 777]),
]


def test_noalloc_backward_equals_workspace_backward_two_calls():
    for i, (N, hq, hkv, hd, dtype, cu) in enumerate(CASES):
        run_case(N, hq, hkv, hd, dtype, cu, seed=900 + i)
    # the large case again, after the smaller one left its statistics behind
    N, hq, hkv, hd, dtype, cu = CASES[0]
    run_case(N, hq, hkv, hd, dtype, cu, seed=900)


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
