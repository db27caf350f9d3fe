"""GPU parity of attention forward and backward against the oracle.

Small cases compare every output element; the benchmark-sized workloads
compare sampled rows (and, for dK/dV, sampled key columns) that the oracle
computes one by one, plus properties that hold at any size.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_close, ensure_library, errors, head_inputs, sample_rows, storage_bytes,
                     to_device, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def pick(t, idx):
    import torch
    return t[torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(t.device)]


def gpu_fwd(q, k, v, scale, causal=True, cu=None):
    import torch
    import ulysses_sp_attention_amd as uly
    N, bs, hq, hd = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((bs, hq, N), float("nan"), dtype=torch.float32, device="cuda")
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    uly.ulysses_attn_fwd(q, k, v, o, lse, scale, causal, cu_t)
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(q, k, v, o, lse, do, scale, causal=True, cu=None):
    import torch
    import ulysses_sp_attention_amd as uly
    N, bs, hq, hd = q.shape
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    code = uly.BF16 if q.dtype == torch.bfloat16 else uly.FP32
    ws = torch.empty(uly.ulysses_attn_bwd_workspace_size(N, bs, hq, k.shape[2], hd, code),
                     dtype=torch.uint8, device="cuda")
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    uly.ulysses_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal, cu_t)
    torch.cuda.synchronize()
    return dq, dk, dv


SMALL = [
    # N, bs, hq, hkv, hd, dtype, causal, cu
    (1, 1, 4, 1, 128, "bf16", True, None),
    (63, 1, 4, 1, 128, "bf16", True, None),
    (64, 1, 4, 1, 128, "bf16", True, None),
    (65, 2, 4, 1, 128, "bf16", True, None),
    (300, 1, 8, 8, 64, "bf16", True, None),
    (257, 1, 2, 1, 128, "bf16", True, None),
    (520, 1, 16, 2, 128, "bf16", True, None),
    (333, 2, 6, 2, 64, "bf16", True, None),
    (200, 1, 4, 1, 128, "bf16", False, None),
    (700, 1, 4, 1, 128, "bf16", True, [0, 1, 65, 130, 131, 500, 700]),
    (400, 1, 4, 2, 64, "bf16", False, [0, 37, 300, 400]),
    (256, 1, 2, 2, 64, "f32", True, None),
    (97, 2, 4, 2, 32, "f32", True, None),
    (150, 1, 4, 1, 128, "f32", True, [0, 50, 51, 150]),
]


def bf16_round(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def to_device_f(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def check_end_to_end(dtype, got, ref, rows=None, cols=None):
    """GPU forward then backward against the exact gradient.  Besides its own
    roundings, the backward sees O rounded to the storage format, so D_i is
    off by up to 2u sum_e |dO_ie| (P|V|)_ie; the oracle's dq_from_D/dk_from_D
    carry that through to dQ and dK."""
    dq, dk, dv = (to_f64(t) for t in got)
    if rows is not None:
        dq = dq[rows]
    if cols is not None:
        dk, dv = dk[cols], dv[cols]
    dq_ref, dk_ref, dv_ref, m = ref
    assert_close(dq, dq_ref, dtype, "dQ (fwd+bwd)", m["dq"] + m["dq_from_D"])
    assert_close(dk, dk_ref, dtype, "dK (fwd+bwd)", m["dk"] + m["dk_from_D"])
    assert_close(dv, dv_ref, dtype, "dV (fwd+bwd)", m["dv"])


def small_inputs(N, bs, hq, hkv, hd, dtype, seed):
    q = synth.normal(seed, 1, (N, bs, hq, hd), dtype=dtype, scale=0.5)
    k = synth.normal(seed, 2, (N, bs, hkv, hd), dtype=dtype)
    v = synth.normal(seed, 3, (N, bs, hkv, hd), dtype=dtype)
    do = synth.normal(seed, 4, (N, bs, hq, hd), dtype=dtype)
    return q, k, v, do


@pytest.mark.parametrize("N,bs,hq,hkv,hd,dtype,causal,cu", SMALL)
def test_fwd_bwd_small_every_element(N, bs, hq, hkv, hd, dtype, causal, cu):
    q, k, v, do = small_inputs(N, bs, hq, hkv, hd, dtype, seed=N + hq)
    scale = 1.0 / np.sqrt(hd)
    qd, kd, vd, dod = (to_device(x, dtype) for x in (q, k, v, do))
    o, lse = gpu_fwd(qd, kd, vd, scale, causal, cu)
    f = [synth.to_f64(x, dtype) for x in (q, k, v, do)]
    o_ref, lse_ref, mo = oracle.attn_fwd(f[0], f[1], f[2], scale, causal, cu, magnitude=True)
    assert_close(to_f64(o), o_ref, dtype, "O", mo)
    assert_close(to_f64(lse), lse_ref, dtype, "LSE")
    # Backward alone: both sides receive the oracle's O (rounded to the storage
    # dtype) and LSE (fp32), so D and P start from the same values.
    o_in = o_ref.astype(np.float32)
    if dtype == "bf16":
        o_in = bf16_round(o_ref)
    lse_in = lse_ref.astype(np.float32)
    dq, dk, dv = gpu_bwd(qd, kd, vd, to_device_f(o_in, dtype), to_device_f(lse_in, "f32"), dod,
                         scale, causal, cu)
    dq_ref, dk_ref, dv_ref, m = oracle.attn_bwd(f[0], f[1], f[2], f[3], scale, causal, cu,
                                                magnitude=True, o=o_in, lse=lse_in)
    assert_close(to_f64(dq), dq_ref, dtype, "dQ", m["dq"])
    assert_close(to_f64(dk), dk_ref, dtype, "dK", m["dk"])
    assert_close(to_f64(dv), dv_ref, dtype, "dV", m["dv"])
    # Forward then backward on the GPU against the exact gradient.
    dq, dk, dv = gpu_bwd(qd, kd, vd, o, lse, dod, scale, causal, cu)
    check_end_to_end(dtype, (dq, dk, dv), oracle.attn_bwd(f[0], f[1], f[2], f[3], scale, causal,
                                                          cu, magnitude=True))


def test_fwd_bwd_are_deterministic():
    q, k, v, do = small_inputs(777, 1, 4, 1, 128, "bf16", seed=5)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    o1, l1 = gpu_fwd(qd, kd, vd, 0.088)
    o2, l2 = gpu_fwd(qd, kd, vd, 0.088)
    assert storage_bytes(o1) == storage_bytes(o2) and storage_bytes(l1) == storage_bytes(l2)
    g1 = gpu_bwd(qd, kd, vd, o1, l1, dod, 0.088)
    g2 = gpu_bwd(qd, kd, vd, o1, l1, dod, 0.088)
    for a, b in zip(g1, g2):
        assert storage_bytes(a) == storage_bytes(b)


@pytest.mark.parametrize("name,n_rand", [("llama8b-share-32k", 1024), ("llama8b-share-128k", 512),
                                          ("long-256k", 256), ("packed-docs-64k", 512)])
def test_fwd_full_size_sampled_rows(name, n_rand):
    w = synth.WORKLOADS[name]
    q, k, v = head_inputs(w)
    cu = w.cu_seqlens()
    qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
    o, lse = gpu_fwd(qd, kd, vd, w.softmax_scale, True, None if cu is None else list(cu))
    rows = sample_rows(w.seqlen, w.seed, n_rand=n_rand)
    f = [synth.to_f64(x, w.dtype) for x in (q, k, v)]
    o_ref, lse_ref, mo = oracle.attn_fwd(f[0], f[1], f[2], w.softmax_scale, True, cu, rows=rows,
                                         magnitude=True)
    assert_close(to_f64(pick(o, rows)), o_ref, w.dtype, "O rows", mo)
    assert_close(to_f64(lse)[:, :, rows], lse_ref, w.dtype, "LSE rows")


def test_bwd_full_size_packed_documents():
    """dQ on sampled rows and dK/dV on whole documents (the last two) plus
    the first keys of the first document, at the packed-document workload."""
    w = synth.WORKLOADS["packed-docs-64k"]
    q, k, v, do = head_inputs(w, (synth.STREAM_Q, synth.STREAM_K, synth.STREAM_V, synth.STREAM_DO))
    cu = w.cu_seqlens()
    qd, kd, vd, dod = (to_device(x, w.dtype) for x in (q, k, v, do))
    o, lse = gpu_fwd(qd, kd, vd, w.softmax_scale, True, list(cu))
    dq, dk, dv = gpu_bwd(qd, kd, vd, o, lse, dod, w.softmax_scale, True, list(cu))
    rows = sample_rows(w.seqlen, w.seed, n_first=128, n_last=128, n_rand=256)
    cols = np.concatenate([np.arange(cu[-3], cu[-1]), np.arange(0, 64)]).astype(np.int64)
    f = [synth.to_f64(x, w.dtype) for x in (q, k, v, do)]
    ref = oracle.attn_bwd(*f, w.softmax_scale, True, cu, dq_rows=rows, dkv_cols=cols, magnitude=True)
    check_end_to_end(w.dtype, (pick(dq, rows), pick(dk, cols), pick(dv, cols)), ref)


def test_bwd_full_size_llama8b_128k():
    """dQ on sampled rows, dK/dV on the last 512 keys (whose visible queries
    the oracle can afford), and the column-sum identity over all keys."""
    w = synth.WORKLOADS["llama8b-share-128k"]
    q, k, v, do = head_inputs(w, (synth.STREAM_Q, synth.STREAM_K, synth.STREAM_V, synth.STREAM_DO))
    qd, kd, vd, dod = (to_device(x, w.dtype) for x in (q, k, v, do))
    o, lse = gpu_fwd(qd, kd, vd, w.softmax_scale)
    dq, dk, dv = gpu_bwd(qd, kd, vd, o, lse, dod, w.softmax_scale)
    rows = sample_rows(w.seqlen, w.seed, n_first=64, n_last=64, n_rand=64)
    cols = np.arange(w.seqlen - 512, w.seqlen, dtype=np.int64)
    f = [synth.to_f64(x, w.dtype) for x in (q, k, v, do)]
    ref = oracle.attn_bwd(*f, w.softmax_scale, True, None, dq_rows=rows, dkv_cols=cols,
                          magnitude=True)
    check_end_to_end(w.dtype, (pick(dq, rows), pick(dk, cols), pick(dv, cols)), ref)
    # sum_j dV_j = sum over the group's heads and all rows of dO (softmax rows sum to 1)
    dv_sum = to_f64(dv).sum(axis=0)[:, 0]
    want = f[3].sum(axis=(0, 2))
    _, rel = errors(dv_sum, want)
    assert rel < 1e-2, rel
