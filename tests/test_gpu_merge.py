"""GPU parity of the partial-result merge (ring / blockwise attention step)
against the oracle, and one ring step built from the forward entry point."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, ensure_library, sample_rows, storage_bytes, to_device, to_f64

pytestmark = pytest.mark.gpu

SEED = 3100


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def partials(N, bs, heads, hd, dtype, seed, lse_scale=20.0, empty=True):
    """Two partial results: O in `dtype` storage, LSE fp32 with some rows -inf."""
    oa = synth.normal(seed, 1, (N, bs, heads, hd), dtype)
    ob = synth.normal(seed, 2, (N, bs, heads, hd), dtype)
    la = synth.normal(seed, 3, (bs, heads, N), "f32", scale=lse_scale)
    lb = synth.normal(seed, 4, (bs, heads, N), "f32", scale=lse_scale)
    if empty:
        la[..., ::7] = -np.inf         # rows where partial a saw no key
        lb[..., ::11] = -np.inf        # ... and b; every 77th row sees none in either
    return oa, la, ob, lb


def gpu_merge(oa, la, ob, lb, dtype, in_place=False):
    import torch
    import ulysses_sp_attention_amd as uly
    ta, tb = to_device(oa, dtype), to_device(ob, dtype)
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    if in_place:
        uly.ulysses_attn_merge(ta, tla, tb, tlb, ta, tla)
        torch.cuda.synchronize()
        return ta, tla
    o = torch.full_like(ta, float("nan"))
    lse = torch.full_like(tla, float("nan"))
    uly.ulysses_attn_merge(ta, tla, tb, tlb, o, lse)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("N,bs,heads,hd,dtype", [
    (257, 2, 3, 128, "bf16"), (100, 1, 4, 64, "bf16"), (33, 1, 2, 32, "bf16"),
    (77, 1, 2, 32, "f32"), (64, 2, 2, 128, "f32"), (1, 1, 1, 64, "f32"),
])
def test_merge_matches_oracle_every_element(N, bs, heads, hd, dtype):
    oa, la, ob, lb = partials(N, bs, heads, hd, dtype, SEED + N)
    o, lse = gpu_merge(oa, la, ob, lb, dtype)
    want_o, want_l = oracle.attn_merge(synth.to_f64(oa, dtype), la, synth.to_f64(ob, dtype), lb)
    got_l = to_f64(lse)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    fin = np.isfinite(want_l)
    assert_close(got_l[fin], want_l[fin], "f32", "LSE")
    assert_close(to_f64(o), want_o, dtype, "O")
    # rows with no key in either partial: exactly zero
    both = np.isneginf(la) & np.isneginf(lb)
    assert both.any()
    got = to_f64(o)
    for b, h, i in zip(*np.nonzero(both)):
        assert np.all(got[i, b, h] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_in_place_equals_out_of_place(dtype):
    oa, la, ob, lb = partials(300, 1, 4, 128 if dtype == "bf16" else 64, dtype, SEED + 7)
    o, lse = gpu_merge(oa, la, ob, lb, dtype)
    oi, lsei = gpu_merge(oa, la, ob, lb, dtype, in_place=True)
    assert storage_bytes(o) == storage_bytes(oi)
    assert storage_bytes(lse) == storage_bytes(lsei)


@pytest.mark.parametrize("n,hq,hkv,hd", [(300, 4, 1, 128), (129, 2, 2, 64)])
def test_ring_step_rebuilds_causal_attention_of_the_second_block(n, hq, hkv, hd):
    """Rows [n, 2n) of causal attention over 2n positions, from two forward
    calls (the first key block fully visible, the second causal) and a merge."""
    import torch
    import ulysses_sp_attention_amd as uly
    seed, scale = SEED + 50 + n, 1.0 / np.sqrt(hd)
    q = synth.normal(seed, synth.STREAM_Q, (2 * n, 1, hq, hd), "bf16")
    k = synth.normal(seed, synth.STREAM_K, (2 * n, 1, hkv, hd), "bf16")
    v = synth.normal(seed, synth.STREAM_V, (2 * n, 1, hkv, hd), "bf16")
    tq, tk, tv = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    parts = []
    for kb, causal in ((slice(0, n), False), (slice(n, 2 * n), True)):
        o = torch.empty_like(tq[n:])
        lse = torch.empty((1, hq, n), dtype=torch.float32, device="cuda")
        uly.ulysses_attn_fwd(tq[n:].contiguous(), tk[kb].contiguous(), tv[kb].contiguous(), o, lse,
                             scale, causal)
        parts.append((o, lse))
    o = torch.empty_like(parts[0][0])
    lse = torch.empty_like(parts[0][1])
    uly.ulysses_attn_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1], o, lse)
    torch.cuda.synchronize()
    want_o, want_l = oracle.attn_fwd(synth.to_f64(q, "bf16"), synth.to_f64(k, "bf16"),
                                     synth.to_f64(v, "bf16"), scale, causal=True,
                                     rows=np.arange(n, 2 * n))
    # each partial LSE comes from the bf16 forward, so the forward's bar applies
    assert_close(to_f64(o), want_o, "bf16", "O")
    assert_close(to_f64(lse), want_l, "bf16", "LSE")


def test_merge_full_size_llama8b_128k_sampled_rows():
    """The 128K rank-share shape (4 heads, hd 128, bf16): every row merged on
    the GPU, sampled rows checked against the oracle."""
    N, bs, heads, hd = 131072, 1, 4, 128
    oa, la, ob, lb = partials(N, bs, heads, hd, "bf16", SEED + 128, lse_scale=8.0)
    o, lse = gpu_merge(oa, la, ob, lb, "bf16")
    rows = sample_rows(N, SEED)
    want_o, want_l = oracle.attn_merge(synth.to_f64(oa[rows], "bf16"), la[..., rows],
                                       synth.to_f64(ob[rows], "bf16"), lb[..., rows])
    got_o, got_l = to_f64(o)[rows], to_f64(lse)[..., rows]
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    fin = np.isfinite(want_l)
    assert_close(got_l[fin], want_l[fin], "f32", "LSE")
    assert_close(got_o, want_o, "bf16", "O")
