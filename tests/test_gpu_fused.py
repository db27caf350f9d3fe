"""The exchange fused into attention: the fused forward and backward must
equal seq_to_head -> attention -> head_to_seq bit for bit (same arithmetic on
the same values; only where rows are read and written differs), must leave
the other ranks' head slots of the output chunks untouched, and must match
the oracle's attention on the rank's head slice of the inputs (the oracle's
own exchange gathers that slice), every element at the small cases and
sampled rows at the 128K share.  Every case runs with the chunks as
consecutive slices of one tensor (the strided-view kernels) and as separate
buffers at descending addresses (the chunk-table kernels)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_close, assert_grads_close, assert_rows_close, ensure_library,
                     sample_rows, storage_bytes, to_device, to_f64)

pytestmark = pytest.mark.gpu

CANARY = 7.0


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def split(t, P):
    n = t.shape[0] // P
    return [t[c * n:(c + 1) * n] for c in range(P)]


LAYOUTS = ["contiguous", "scattered"]


def place(t, P, layout):
    """P chunks holding t's sequence slices: views of t itself, or copies in
    one buffer in reverse order with a gap (no chunk follows its predecessor)."""
    if layout == "contiguous":
        return split(t, P)
    import torch
    n = t.shape[0] // P
    buf = torch.empty(((P + 1) * n,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    chunks = [buf[(P - c) * n:(P - c + 1) * n] for c in range(P)]
    for c in range(P):
        chunks[c].copy_(t[c * n:(c + 1) * n])
    return chunks


def gather(chunks):
    import torch
    return torch.cat(list(chunks), dim=0)


def local_heads(heads, P):
    return heads // P if heads >= P else 1


def rank_inputs(host, P, rank):
    """The rank's head-sharded inputs by the oracle's exchange, from float64
    host copies [N, bs, H, hd] of the sequence-sharded tensors."""
    n = host[0].shape[0] // P
    return [oracle.seq_to_head([np.ascontiguousarray(x[c * n:(c + 1) * n]) for c in range(P)], rank)
            for x in host]


def rank_slice(t, P, rank, rows=None):
    """This rank's head slots of a gathered [N, bs, H, hd] output, float64."""
    hl = t.shape[2] // P
    out = t[:, :, rank * hl:(rank + 1) * hl]
    if rows is not None:
        import torch
        out = out[torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(t.device)]
    return to_f64(out)


_ORACLE_CACHE = {}


def head_slices(tensors, P, rank):
    """The rank's head slice of full-size device tensors [N, bs, H, hd] by
    plain indexing, float64 (at the 128K share, float64 copies of every head
    would take 10 GB of host memory); H >= P here, so no head is replicated."""
    out = []
    for t in tensors:
        hl = t.shape[2] // P
        out.append(to_f64(t[:, :, rank * hl:(rank + 1) * hl]))
    return out


def oracle_fwd(key, host, P, rank, scale, causal, cu, rows=None, sliced=False):
    """oracle.attn_fwd on the rank's slice (cached per key: both layouts of a
    case compare with the same values).  host: float64 copies of the
    sequence-sharded inputs, or (sliced) of the rank's head slice."""
    if key not in _ORACLE_CACHE:
        ql, kl, vl = host[:3] if sliced else rank_inputs(host[:3], P, rank)
        _ORACLE_CACHE[key] = oracle.attn_fwd(ql, kl, vl, scale, causal, cu, rows=rows,
                                             magnitude=True)
    return _ORACLE_CACHE[key]


def oracle_bwd(key, host, P, rank, scale, causal, cu, rows=None, cols=None, sliced=False):
    if key not in _ORACLE_CACHE:
        ql, kl, vl, dol = host if sliced else rank_inputs(host, P, rank)
        _ORACLE_CACHE[key] = oracle.attn_bwd(ql, kl, vl, dol, scale, causal, cu, dq_rows=rows,
                                             dkv_cols=cols, magnitude=True)
    return _ORACLE_CACHE[key]


def unfused_fwd(qc, kc, vc, rank, scale, causal, cu_t, o_full):
    """Reference: the three separate calls."""
    import torch
    import ulysses_sp_attention_amd as uly
    P = len(qc)
    n, bs, hq, hd = qc[0].shape
    hkv = kc[0].shape[2]
    N = P * n
    qh = torch.empty((N, bs, hq // P, hd), dtype=qc[0].dtype, device="cuda")
    kh = torch.empty((N, bs, local_heads(hkv, P), hd), dtype=qc[0].dtype, device="cuda")
    vh = torch.empty_like(kh)
    uly.ulysses_seq_to_head(qc, rank, qh)
    uly.ulysses_seq_to_head(kc, rank, kh)
    uly.ulysses_seq_to_head(vc, rank, vh)
    o = torch.empty_like(qh)
    lse = torch.empty((bs, hq // P, N), dtype=torch.float32, device="cuda")
    uly.ulysses_attn_fwd(qh, kh, vh, o, lse, scale, causal, cu_t)
    uly.ulysses_head_to_seq(o, rank, split(o_full, P))
    return lse


FWD_CASES = [
    # P, rank, n_local, bs, hq, hkv, hd, causal, cu
    (2, 1, 64, 1, 4, 4, 64, True, None),
    (4, 2, 128, 2, 8, 2, 128, True, None),      # fewer kv heads than ranks: replicated
    (4, 3, 64, 1, 8, 4, 128, False, None),
    (8, 3, 128, 1, 32, 8, 128, True, None),     # the Llama-8B head counts
    (4, 0, 192, 1, 8, 8, 64, True, [0, 100, 101, 400, 768]),
    (16, 15, 64, 1, 16, 16, 128, True, None),   # the largest P of the fused calls
    (3, 1, 64, 1, 6, 3, 128, True, [0, 64, 130, 192]),
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("P,rank,n,bs,hq,hkv,hd,causal,cu", FWD_CASES)
def test_fused_fwd_equals_exchange_attention_exchange(P, rank, n, bs, hq, hkv, hd, causal, cu,
                                                      layout):
    import torch
    N, seed, scale = P * n, 4200 + P * 7 + rank, 1.0 / np.sqrt(hd)
    q = to_device(synth.normal(seed, synth.STREAM_Q, (N, bs, hq, hd), "bf16"), "bf16")
    k = to_device(synth.normal(seed, synth.STREAM_K, (N, bs, hkv, hd), "bf16"), "bf16")
    v = to_device(synth.normal(seed, synth.STREAM_V, (N, bs, hkv, hd), "bf16"), "bf16")
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    o, lse = check_fwd(q, k, v, P, rank, scale, causal, cu_t, layout)
    host = [to_f64(t) for t in (q, k, v)]
    o_ref, lse_ref, mo = oracle_fwd(("fwd", P, rank, n, bs, hq, hkv, hd, causal, str(cu)), host, P,
                                    rank, scale, causal, cu)
    got = rank_slice(o, P, rank)
    assert_close(got, o_ref, "bf16", "O (fused) against the oracle", mo)
    assert_rows_close(got, o_ref, "bf16", "O rows (fused) against the oracle")
    assert_close(to_f64(lse), lse_ref, "bf16", "LSE (fused) against the oracle")


def check_fwd(q, k, v, P, rank, scale, causal, cu_t, layout):
    import torch
    import ulysses_sp_attention_amd as uly
    hq = q.shape[2]
    o_ref = torch.full_like(q, CANARY)
    lse_ref = unfused_fwd(split(q, P), split(k, P), split(v, P), rank, scale, causal, cu_t, o_ref)
    oc = place(torch.full_like(q, CANARY), P, layout)
    lse = torch.full_like(lse_ref, float("nan"))
    uly.ulysses_attn_fwd_fused(place(q, P, layout), place(k, P, layout), place(v, P, layout), oc,
                               lse, rank, scale, causal, cu_t)
    torch.cuda.synchronize()
    o = gather(oc)
    assert storage_bytes(o) == storage_bytes(o_ref)      # other ranks' slots keep the canary
    assert storage_bytes(lse) == storage_bytes(lse_ref)
    hl = hq // P
    untouched = torch.cat([o[:, :, :rank * hl], o[:, :, (rank + 1) * hl:]], dim=2)
    assert bool(torch.all(untouched == CANARY))
    return o, lse


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fused_fwd_full_size_llama8b_128k(layout):
    """The benchmark's shape: P = 8 chunks of 16384 tokens, 32 q / 8 kv heads, rank 3."""
    w = synth.WORKLOADS["llama8b-share-128k"]
    P, rank, N = w.P, w.rank, w.seqlen
    q, k, v = (to_device(w.seq_tensor(st, heads, scale), "bf16")
               for st, heads, scale in ((synth.STREAM_Q, w.hq, w.q_prescale),
                                        (synth.STREAM_K, w.hkv, 1.0), (synth.STREAM_V, w.hkv, 1.0)))
    o, lse = check_fwd(q, k, v, P, rank, w.softmax_scale, True, None, layout)
    rows = sample_rows(N, w.seed, n_first=64, n_last=64, n_rand=192)
    if ("fwd128k",) not in _ORACLE_CACHE:
        host = head_slices((q, k, v), P, rank)
    else:
        host = None
    o_ref, lse_ref, mo = oracle_fwd(("fwd128k",), host, P, rank, w.softmax_scale, True, None,
                                    rows=rows, sliced=True)
    got = rank_slice(o, P, rank, rows)
    assert_close(got, o_ref, "bf16", "O rows (fused, 128K) against the oracle", mo)
    assert_rows_close(got, o_ref, "bf16", "O per row (fused, 128K) against the oracle")
    assert_close(to_f64(lse)[:, :, rows], lse_ref, "bf16", "LSE rows (fused, 128K) against the oracle")


def unfused_bwd(qc, kc, vc, oc, lse, doc, rank, scale, causal, cu_t, dq_full, dk_full, dv_full):
    """Reference: dO to the head layout, the backward, dQ/dK/dV back."""
    import torch
    import ulysses_sp_attention_amd as uly
    P = len(qc)
    n, bs, hq, hd = qc[0].shape
    hkv = kc[0].shape[2]
    N = P * n
    heads = lambda h: torch.empty((N, bs, h, hd), dtype=qc[0].dtype, device="cuda")
    qh, oh, doh = heads(hq // P), heads(hq // P), heads(hq // P)
    kh, vh = heads(hkv // P), heads(hkv // P)
    for chunks, h in ((qc, qh), (kc, kh), (vc, vh), (oc, oh), (doc, doh)):
        uly.ulysses_seq_to_head(chunks, rank, h)
    dqh, dkh, dvh = torch.empty_like(qh), torch.empty_like(kh), torch.empty_like(vh)
    ws = workspace(N, bs, hq // P, hkv // P, hd)
    uly.ulysses_attn_bwd(qh, kh, vh, oh, lse, doh, dqh, dkh, dvh, ws, scale, causal, cu_t)
    for h, full in ((dqh, dq_full), (dkh, dk_full), (dvh, dv_full)):
        uly.ulysses_head_to_seq(h, rank, split(full, P))


def workspace(N, bs, hq_l, hkv_l, hd):
    import torch
    import ulysses_sp_attention_amd as uly
    nbytes = uly.ulysses_attn_bwd_workspace_size(N, bs, hq_l, hkv_l, hd, uly.BF16)
    # contents on entry must not matter: start from garbage
    return torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")


def check_bwd(q, k, v, do, P, rank, scale, causal, cu_t, layout):
    """Forward (fused), then the fused backward against the unfused chain."""
    import torch
    import ulysses_sp_attention_amd as uly
    N, bs, hq, hd = q.shape
    hkv = k.shape[2]
    o = torch.full_like(q, CANARY)
    lse = torch.empty((bs, hq // P, N), dtype=torch.float32, device="cuda")
    uly.ulysses_attn_fwd_fused(split(q, P), split(k, P), split(v, P), split(o, P), lse, rank,
                               scale, causal, cu_t)
    ref = [torch.full_like(t, CANARY) for t in (q, k, v)]
    unfused_bwd(split(q, P), split(k, P), split(v, P), split(o, P), lse, split(do, P), rank, scale,
                causal, cu_t, *ref)
    outs = [place(torch.full_like(t, CANARY), P, layout) for t in (q, k, v)]
    ws = workspace(N, bs, hq // P, hkv // P, hd)
    uly.ulysses_attn_bwd_fused(*[place(t, P, layout) for t in (q, k, v, o)], lse,
                               place(do, P, layout), *outs, ws, rank, scale, causal, cu_t)
    torch.cuda.synchronize()
    for name, oc, r, heads in zip(("dq", "dk", "dv"), outs, ref, (hq, hkv, hkv)):
        g = gather(oc)
        assert torch.equal(g.view(torch.int16), r.view(torch.int16)), name
        hl = heads // P
        untouched = torch.cat([g[:, :, :rank * hl], g[:, :, (rank + 1) * hl:]], dim=2)
        assert bool(torch.all(untouched == CANARY)), name
    return [gather(oc) for oc in outs]


BWD_CASES = [
    # P, rank, n_local, bs, hq, hkv, hd, causal, cu
    (2, 1, 64, 1, 4, 4, 64, True, None),
    (4, 2, 128, 2, 8, 4, 128, True, None),
    (4, 3, 64, 1, 8, 4, 128, False, None),
    (8, 3, 128, 1, 32, 8, 128, True, None),     # the Llama-8B head counts
    (4, 0, 192, 1, 8, 8, 64, True, [0, 100, 101, 400, 768]),
    (16, 15, 64, 1, 16, 16, 128, True, None),   # the largest P of the fused calls
    (3, 1, 64, 1, 6, 3, 128, True, [0, 64, 130, 192]),
    (2, 0, 320, 1, 16, 2, 128, True, [0, 1, 2, 333, 640]),   # group of 8 q heads per kv head
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("P,rank,n,bs,hq,hkv,hd,causal,cu", BWD_CASES)
def test_fused_bwd_equals_exchange_backward_exchange(P, rank, n, bs, hq, hkv, hd, causal, cu,
                                                     layout):
    import torch
    N, seed, scale = P * n, 5200 + P * 7 + rank, 1.0 / np.sqrt(hd)
    q = to_device(synth.normal(seed, synth.STREAM_Q, (N, bs, hq, hd), "bf16"), "bf16")
    k = to_device(synth.normal(seed, synth.STREAM_K, (N, bs, hkv, hd), "bf16"), "bf16")
    v = to_device(synth.normal(seed, synth.STREAM_V, (N, bs, hkv, hd), "bf16"), "bf16")
    do = to_device(synth.normal(seed, synth.STREAM_DO, (N, bs, hq, hd), "bf16"), "bf16")
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    dq, dk, dv = check_bwd(q, k, v, do, P, rank, scale, causal, cu_t, layout)
    host = [to_f64(t) for t in (q, k, v, do)]
    ref = oracle_bwd(("bwd", P, rank, n, bs, hq, hkv, hd, causal, str(cu)), host, P, rank, scale,
                     causal, cu)
    assert_grads_close("bf16", rank_slice(dq, P, rank), rank_slice(dk, P, rank),
                       rank_slice(dv, P, rank), ref, "fused, against the oracle")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fused_bwd_full_size_llama8b_128k(layout):
    """The benchmark's shape: P = 8 chunks of 16384 tokens, 32 q / 8 kv heads, rank 3."""
    w = synth.WORKLOADS["llama8b-share-128k"]
    P, rank, N = w.P, w.rank, w.seqlen
    q, k, v, do = (to_device(w.seq_tensor(st, heads, scale), "bf16")
                   for st, heads, scale in ((synth.STREAM_Q, w.hq, w.q_prescale),
                                            (synth.STREAM_K, w.hkv, 1.0),
                                            (synth.STREAM_V, w.hkv, 1.0),
                                            (synth.STREAM_DO, w.hq, 1.0)))
    dq, dk, dv = check_bwd(q, k, v, do, P, rank, w.softmax_scale, True, None, layout)
    # dQ on sampled rows, dK/dV on the last 256 keys (whose visible queries the
    # oracle can afford)
    rows = sample_rows(N, w.seed, n_first=32, n_last=32, n_rand=32)
    cols = np.arange(N - 256, N, dtype=np.int64)
    host = head_slices((q, k, v, do), P, rank) if ("bwd128k",) not in _ORACLE_CACHE else None
    ref = oracle_bwd(("bwd128k",), host, P, rank, w.softmax_scale, True, None, rows=rows, cols=cols,
                     sliced=True)
    assert_grads_close("bf16", rank_slice(dq, P, rank, rows), rank_slice(dk, P, rank, cols),
                       rank_slice(dv, P, rank, cols), ref, "fused, 128K, against the oracle")
