"""The sequence-tiled SwiGLU MLP against the oracle, element by element.

The GPU keeps g, u and da in fp32 and rounds a, dg and du to bf16 as GEMM
operands (relative 2^-9 each); y and dx are rounded to bf16 once, the weight
gradients stay fp32.  With the oracle's magnitudes (|a||Wd|^T, |dg||Wg| +
|du||Wu|, |dg|^T|x|, |du|^T|x|, |dy|^T|a|) the bars are
  y, dx          : 2^-7 magnitude + 2^-8 |value|
  dWg, dWu, dWd  : 2^-7 magnitude
(twice the operand rounding, which also covers the fp32 sums).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import ensure_library, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def weights(seed, d, inter):
    wg = synth.normal(seed, synth.STREAM_MLP_GATE, (inter, d), "bf16", scale=1 / np.sqrt(d))
    wu = synth.normal(seed, synth.STREAM_MLP_UP, (inter, d), "bf16", scale=1 / np.sqrt(d))
    wd = synth.normal(seed, synth.STREAM_MLP_DOWN, (d, inter), "bf16", scale=1 / np.sqrt(inter))
    return wg, wu, wd


def f64(b):
    return synth.to_f64(b, "bf16")


def run_gpu(x, wg, wu, wd, dy, shard):
    import torch
    import ulysses_sp_attention_amd as uly
    T, d = x.shape
    inter = wg.shape[0]
    dev = [to_device(a, "bf16") for a in (x, wg, wu, wd, dy)]
    y = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dx = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dwg = torch.full((inter, d), float("nan"), device="cuda")
    dwu = torch.full((inter, d), float("nan"), device="cuda")
    dwd = torch.full((d, inter), float("nan"), device="cuda")
    s = max(min(shard, T), 1)
    ws_f = torch.full((uly.ulysses_tiled_mlp_workspace_size(s, d, inter, False) // 4,),
                      float("nan"), device="cuda")
    ws_b = torch.full((uly.ulysses_tiled_mlp_workspace_size(s, d, inter, True) // 4,),
                      float("nan"), device="cuda")
    uly.ulysses_tiled_mlp_fwd(dev[0], dev[1], dev[2], dev[3], y, ws_f, shard)
    uly.ulysses_tiled_mlp_bwd(*dev, dx, dwg, dwu, dwd, ws_b, shard)
    torch.cuda.synchronize()
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    return host(y), host(dx), host(dwg), host(dwu), host(dwd)


def check(got, ref, mags, rows=None):
    names = ("y", "dx", "dwg", "dwu", "dwd")
    for i, (n, g, r) in enumerate(zip(names, got, ref)):
        if rows is not None and n in ("y", "dx"):
            g = g[rows]
        tol = 2.0 ** -7 * mags[n] + (2.0 ** -8 * np.abs(r) if n in ("y", "dx") else 0.0)
        err = np.abs(g - r)
        assert np.all(err <= tol), (n, float(np.max(err - tol)))


CASES = [
    # T, d, inter, shard
    (100, 64, 176, 32),      # ragged last shard
    (37, 128, 352, 16),
    (64, 64, 64, 64),        # one shard
    (130, 32, 96, 200),      # shard larger than T
    (3, 8, 8, 1),            # one row per shard
]


@pytest.mark.parametrize("T,d,inter,shard", CASES)
def test_tiled_mlp_matches_oracle(T, d, inter, shard):
    seed = 8000 + T + d + inter
    x = synth.normal(seed, synth.STREAM_HIDDEN, (T, d), "bf16")
    dy = synth.normal(seed, synth.STREAM_DO, (T, d), "bf16")
    wg, wu, wd = weights(seed, d, inter)
    ref = oracle.swiglu_mlp(f64(x), f64(wg), f64(wu), f64(wd), f64(dy), magnitude=True)
    check(run_gpu(x, wg, wu, wd, dy, shard), ref[:5], ref[5])


def test_tiled_mlp_shard_size_does_not_change_results():
    """Rows are independent and the weight gradients sum shards in order:
    y and dx are bitwise the same for any shard size; dW agree to fp32
    summation order."""
    x = synth.normal(5, synth.STREAM_HIDDEN, (96, 64), "bf16")
    dy = synth.normal(5, synth.STREAM_DO, (96, 64), "bf16")
    wg, wu, wd = weights(5, 64, 128)
    a = run_gpu(x, wg, wu, wd, dy, 96)
    b = run_gpu(x, wg, wu, wd, dy, 24)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for ga, gb in zip(a[2:], b[2:]):
        np.testing.assert_allclose(ga, gb, rtol=1e-5, atol=1e-6)


def test_tiled_mlp_empty_input():
    wg, wu, wd = weights(1, 16, 32)
    _, _, dwg, dwu, dwd = run_gpu(np.zeros((0, 16), np.uint16), wg, wu, wd,
                                  np.zeros((0, 16), np.uint16), 8)
    assert not dwg.any() and not dwu.any() and not dwd.any()


def test_tiled_mlp_full_size_llama8b_sampled():
    """The Llama-8B MLP (d = 4096, inter = 14336) over one rank's 16384 tokens
    in ceil(T / d) = 4 shards.  y on sampled rows against the oracle on those
    rows; the backward with dy zero except on the sampled rows, so that dx on
    those rows and every weight gradient (a sum over the sampled rows only)
    are checked whole against the oracle."""
    import torch
    import ulysses_sp_attention_amd as uly
    T, d, inter, seed = 16384, 4096, 14336, 77
    sample = [0, 1, 4095, 4096, 9000, 12288, T - 1]
    x = synth.normal(seed, synth.STREAM_HIDDEN, (T, d), "bf16")
    dy = np.zeros((T, d), np.uint16)
    dy[sample] = synth.normal(seed, synth.STREAM_DO, (len(sample), d), "bf16")
    wg, wu, wd = weights(seed, d, inter)
    got = run_gpu(x, wg, wu, wd, dy, d)
    ref = oracle.swiglu_mlp(f64(x[sample]), f64(wg), f64(wu), f64(wd), f64(dy[sample]),
                            magnitude=True)
    check(got, ref[:5], ref[5], rows=sample)
    del got
    torch.cuda.empty_cache()
