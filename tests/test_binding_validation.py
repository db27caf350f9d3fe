"""The Python binding checks every tensor before it calls the library (CPU
only; nothing is launched).

The library sees only pointers and sizes, so the binding must refuse what
would make a kernel touch memory it does not own: a host tensor, a
non-contiguous view, a buffer of the wrong shape (too small to write, or
read past its end) or of the wrong element type.  These tests replace the
library loader with a stub that records the call and the device check with
one that accepts CPU tensors, so that shapes, types and layouts can be
exercised here: every valid call must reach the stub, every broken one must
raise ValueError first.
"""
import pytest
import torch

import ulysses_sp_attention_amd as uly

BF = torch.bfloat16
F32 = torch.float32


class Reached(Exception):
    """The binding got past its checks and asked for the library."""


@pytest.fixture
def stub(monkeypatch):
    def no_library(*a, **k):
        raise Reached()
    monkeypatch.setattr(uly, "load_library", no_library)
    monkeypatch.setattr(uly, "_device_ok", lambda t: True)
    monkeypatch.setattr(uly, "_stream", lambda s: 0)


def e(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def chunks(P, n, bs, h, hd, dtype=BF):
    return [e(n, bs, h, hd, dtype=dtype) for _ in range(P)]


def noncontig(*shape, dtype=BF):
    """A non-contiguous view of the given shape."""
    t = torch.zeros(tuple(shape[:-2]) + (shape[-1], shape[-2]), dtype=dtype)
    return t.transpose(-1, -2)


# Valid arguments of every entry point: P=2, n_local=8, bs=1, 4 q / 2 kv heads, hd=64.
P, n, bs, hq, hkv, hd = 2, 8, 1, 4, 2, 64
N = P * n


def valid(name):
    if name == "seq_to_head":
        return dict(chunks=chunks(P, n, bs, hq, hd), rank=0, out=e(N, bs, hq // P, hd))
    if name == "head_to_seq":
        return dict(inp=e(N, bs, hq // P, hd), rank=0, chunks=chunks(P, n, bs, hq, hd))
    if name == "seq_to_head_batch":
        return dict(pairs=[(chunks(P, n, bs, hq, hd), e(N, bs, hq // P, hd)),
                           (chunks(P, n, bs, hkv, hd), e(N, bs, hkv // P, hd))], rank=1)
    if name == "attn_fwd":
        return dict(q=e(N, bs, hq, hd), k=e(N, bs, hkv, hd), v=e(N, bs, hkv, hd), o=e(N, bs, hq, hd),
                    lse=e(bs, hq, N, dtype=F32), softmax_scale=0.125, causal=True,
                    cu_seqlens=torch.tensor([0, 5, N], dtype=torch.int32))
    if name == "attn_bwd":
        return dict(q=e(N, bs, hq, hd), k=e(N, bs, hkv, hd), v=e(N, bs, hkv, hd), o=e(N, bs, hq, hd),
                    lse=e(bs, hq, N, dtype=F32), dout=e(N, bs, hq, hd), dq=e(N, bs, hq, hd),
                    dk=e(N, bs, hkv, hd), dv=e(N, bs, hkv, hd), workspace=e(4096, dtype=torch.uint8),
                    softmax_scale=0.125)
    if name == "attn_merge":
        return dict(o_a=e(N, bs, hq, hd), lse_a=e(bs, hq, N, dtype=F32), o_b=e(N, bs, hq, hd),
                    lse_b=e(bs, hq, N, dtype=F32), o=e(N, bs, hq, hd), lse=e(bs, hq, N, dtype=F32))
    if name == "attn_fwd_fused":
        return dict(q_chunks=chunks(P, n, bs, hq, hd), k_chunks=chunks(P, n, bs, hkv, hd),
                    v_chunks=chunks(P, n, bs, hkv, hd), o_chunks=chunks(P, n, bs, hq, hd),
                    lse=e(bs, hq // P, N, dtype=F32), rank=1, softmax_scale=0.125)
    if name == "attn_bwd_fused":
        return dict(q_chunks=chunks(P, n, bs, hq, hd), k_chunks=chunks(P, n, bs, hkv, hd),
                    v_chunks=chunks(P, n, bs, hkv, hd), o_chunks=chunks(P, n, bs, hq, hd),
                    lse=e(bs, hq // P, N, dtype=F32), do_chunks=chunks(P, n, bs, hq, hd),
                    dq_chunks=chunks(P, n, bs, hq, hd), dk_chunks=chunks(P, n, bs, hkv, hd),
                    dv_chunks=chunks(P, n, bs, hkv, hd), workspace=e(4096, dtype=torch.uint8),
                    rank=0, softmax_scale=0.125)
    if name == "logits_loss":
        T, d, V = 6, 16, 40
        return dict(h=e(T, d), w=e(V, d), labels=e(T, dtype=torch.int64), loss_rows=e(T, dtype=F32),
                    loss_sum=e(1, dtype=F32), n_good=e(1, dtype=torch.int64), dh=e(T, d),
                    dw=e(V, d, dtype=F32), workspace=e(4096, dtype=torch.uint8))
    if name == "tiled_mlp_fwd":
        T, d, I = 6, 16, 24
        return dict(x=e(T, d), wg=e(I, d), wu=e(I, d), wd=e(d, I), y=e(T, d),
                    workspace=e(4096, dtype=torch.uint8))
    if name == "tiled_mlp_bwd":
        T, d, I = 6, 16, 24
        return dict(x=e(T, d), wg=e(I, d), wu=e(I, d), wd=e(d, I), dy=e(T, d), dx=e(T, d),
                    dwg=e(I, d, dtype=F32), dwu=e(I, d, dtype=F32), dwd=e(d, I, dtype=F32),
                    workspace=e(4096, dtype=torch.uint8))
    raise KeyError(name)


ENTRY = {
    "seq_to_head": uly.ulysses_seq_to_head, "head_to_seq": uly.ulysses_head_to_seq,
    "seq_to_head_batch": uly.ulysses_seq_to_head_batch, "attn_fwd": uly.ulysses_attn_fwd,
    "attn_bwd": uly.ulysses_attn_bwd, "attn_merge": uly.ulysses_attn_merge,
    "attn_fwd_fused": uly.ulysses_attn_fwd_fused, "attn_bwd_fused": uly.ulysses_attn_bwd_fused,
    "logits_loss": uly.ulysses_logits_loss, "tiled_mlp_fwd": uly.ulysses_tiled_mlp_fwd,
    "tiled_mlp_bwd": uly.ulysses_tiled_mlp_bwd,
}


@pytest.mark.parametrize("name", sorted(ENTRY))
def test_valid_arguments_reach_the_library(stub, name):
    with pytest.raises(Reached):
        ENTRY[name](**valid(name))


# (entry point, argument, replacement, expected message fragment)
BROKEN = [
    ("seq_to_head", "out", lambda: e(N - 1, bs, hq // P, hd), "shape"),        # one row short
    ("seq_to_head", "out", lambda: e(N, bs, hq // P, hd, dtype=F32), "dtype"),
    ("seq_to_head", "chunks", lambda: chunks(P, n, bs, hq, hd)[:1] + [e(n + 1, bs, hq, hd)], "shape"),
    ("head_to_seq", "inp", lambda: noncontig(N, bs, hq // P, hd), "contiguous"),
    ("head_to_seq", "inp", lambda: e(N, bs, hq, hd), "shape"),                 # all heads
    ("seq_to_head_batch", "pairs", lambda: [(chunks(P, n, bs, hq, hd), e(N, bs, hq, hd))], "shape"),
    ("seq_to_head_batch", "pairs", lambda: [], "non-empty"),
    ("attn_fwd", "k", lambda: noncontig(N, bs, hkv, hd), "contiguous"),
    ("attn_fwd", "v", lambda: e(N, bs, hq, hd), "shape"),
    ("attn_fwd", "o", lambda: e(N // 2, bs, hq, hd), "shape"),
    ("attn_fwd", "lse", lambda: e(bs, hq, N), "dtype"),
    ("attn_fwd", "lse", lambda: e(bs, hq, N - 1, dtype=F32), "shape"),
    ("attn_fwd", "cu_seqlens", lambda: torch.tensor([0, N], dtype=torch.int64), "dtype"),
    ("attn_fwd", "cu_seqlens", lambda: torch.tensor([N], dtype=torch.int32), "offsets"),
    ("attn_fwd", "q", lambda: e(N, hq, hd), "4-D"),
    ("attn_bwd", "dq", lambda: e(N, bs, hkv, hd), "shape"),                   # undersized
    ("attn_bwd", "dout", lambda: e(N, bs, hq, hd, dtype=F32), "dtype"),
    ("attn_bwd", "workspace", lambda: noncontig(64, 64, dtype=torch.uint8), "contiguous"),
    ("attn_merge", "lse_b", lambda: e(bs, hq, N + 1, dtype=F32), "shape"),
    ("attn_merge", "o", lambda: e(N, bs, hq, hd, dtype=F32), "dtype"),
    ("attn_fwd_fused", "v_chunks", lambda: chunks(P, n + 64, bs, hkv, hd), "v_chunks"),
    ("attn_fwd_fused", "o_chunks", lambda: chunks(P, n, bs, hkv, hd), "heads"),
    ("attn_fwd_fused", "lse", lambda: e(bs, hq, N, dtype=F32), "shape"),
    ("attn_bwd_fused", "dk_chunks", lambda: chunks(P, n, bs, hq, hd), "heads"),
    ("attn_bwd_fused", "do_chunks", lambda: chunks(P + 1, n, bs, hq, hd), "do_chunks"),
    ("logits_loss", "labels", lambda: e(6, dtype=torch.int32), "dtype"),
    ("logits_loss", "dw", lambda: e(40, 16), "dtype"),
    ("logits_loss", "dh", lambda: e(5, 16), "shape"),
    ("tiled_mlp_fwd", "wd", lambda: e(24, 16), "shape"),                      # transposed
    ("tiled_mlp_fwd", "y", lambda: noncontig(6, 16), "contiguous"),
    ("tiled_mlp_bwd", "dwd", lambda: e(24, 16, dtype=F32), "shape"),
    ("tiled_mlp_bwd", "dx", lambda: e(6, 16, dtype=F32), "dtype"),
]


@pytest.mark.parametrize("name,arg,bad,msg", BROKEN,
                         ids=[f"{b[0]}-{b[1]}-{i}" for i, b in enumerate(BROKEN)])
def test_broken_arguments_raise_before_the_library(stub, name, arg, bad, msg):
    kw = valid(name)
    kw[arg] = bad()
    with pytest.raises(ValueError, match=msg):
        ENTRY[name](**kw)


@pytest.mark.parametrize("name", sorted(ENTRY))
def test_host_tensors_are_refused(monkeypatch, name):
    """With the real device check, CPU tensors never reach the library."""
    def no_library(*a, **k):
        raise Reached()
    monkeypatch.setattr(uly, "load_library", no_library)
    with pytest.raises(ValueError, match="current GPU"):
        ENTRY[name](**valid(name))
