"""The whole rank-share path on the GPU, every rank of an emulated P-rank job:
seq_to_head -> attention forward -> head_to_seq, and for the backward
seq_to_head(dO) -> attention backward -> head_to_seq(dQ, dK, dV).
Because heads are independent, assembling every rank's share must reproduce
full multi-head attention (and its gradients) over all heads."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, ensure_library, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def run_all_ranks(w: synth.Workload, N: int):
    import torch
    import ulysses_sp_attention_amd as uly
    P, n = w.P, N // w.P
    hl, kl = w.hq // P, w.hkv // P
    gen = {s: synth.normal(w.seed, s, (N, w.bs, heads, w.head_dim), dtype=w.dtype,
                           scale=w.q_prescale if s == synth.STREAM_Q else 1.0)
           for s, heads in ((synth.STREAM_Q, w.hq), (synth.STREAM_K, w.hkv), (synth.STREAM_V, w.hkv),
                            (synth.STREAM_DO, w.hq))}
    dev = {s: to_device(x, w.dtype) for s, x in gen.items()}
    chunks = {s: [t[c * n:(c + 1) * n] for c in range(P)] for s, t in dev.items()}
    outs = {name: torch.full((N, w.bs, heads, w.head_dim), float("nan"), dtype=dev[1].dtype,
                             device="cuda")
            for name, heads in (("o", w.hq), ("dq", w.hq), ("dk", w.hkv), ("dv", w.hkv))}
    out_chunks = {k: [t[c * n:(c + 1) * n] for c in range(P)] for k, t in outs.items()}
    code = uly.BF16 if w.dtype == "bf16" else uly.FP32
    for r in range(P):
        loc = {}
        for s, heads in ((synth.STREAM_Q, hl), (synth.STREAM_K, kl), (synth.STREAM_V, kl),
                         (synth.STREAM_DO, hl)):
            loc[s] = torch.empty((N, w.bs, heads, w.head_dim), dtype=dev[1].dtype, device="cuda")
            uly.ulysses_seq_to_head(chunks[s], r, loc[s])
        q, k, v, do = (loc[s] for s in (1, 2, 3, 4))
        o = torch.empty_like(q)
        lse = torch.empty((w.bs, hl, N), dtype=torch.float32, device="cuda")
        uly.ulysses_attn_fwd(q, k, v, o, lse, w.softmax_scale, True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(uly.ulysses_attn_bwd_workspace_size(N, w.bs, hl, kl, w.head_dim, code),
                         dtype=torch.uint8, device="cuda")
        uly.ulysses_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.softmax_scale, True)
        for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            uly.ulysses_head_to_seq(t, r, out_chunks[name])
    torch.cuda.synchronize()
    return gen, outs


@pytest.mark.parametrize("name,N", [("tiny-p2", 256), ("llama8b-share-32k", 1024)])
def test_all_ranks_assemble_full_multi_head_attention(name, N):
    w = synth.WORKLOADS[name]
    gen, outs = run_all_ranks(w, N)
    f = {s: synth.to_f64(x, w.dtype) for s, x in gen.items()}
    o_ref, _, mo = oracle.attn_fwd(f[1], f[2], f[3], w.softmax_scale, True, magnitude=True)
    assert_close(to_f64(outs["o"]), o_ref, w.dtype, "O", mo)
    # forward then backward against the exact gradient: D sees O rounded to
    # the storage format (see test_gpu_attention.check_end_to_end)
    dq_ref, dk_ref, dv_ref, m = oracle.attn_bwd(f[1], f[2], f[3], f[4], w.softmax_scale, True,
                                                magnitude=True)
    assert_close(to_f64(outs["dq"]), dq_ref, w.dtype, "dQ", m["dq"], d_mag=m["dq_from_D"])
    assert_close(to_f64(outs["dk"]), dk_ref, w.dtype, "dK", m["dk"], k_u=3, d_mag=m["dk_from_D"])
    assert_close(to_f64(outs["dv"]), dv_ref, w.dtype, "dV", m["dv"])
    assert not any(np.isnan(to_f64(t)).any() for t in outs.values())
