"""GPU parity of the layout exchange against the oracle: bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from helpers import ensure_library, host_storage, storage_bytes, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def run_seq_to_head(chunks_host, rank, dtype):
    import torch
    import ulysses_sp_attention_amd as uly
    dev = [to_device(c, dtype) for c in chunks_host]
    n, bs, heads, hd = chunks_host[0].shape
    P = len(chunks_host)
    hl = heads // P if heads >= P else 1
    out = torch.full((P * n, bs, hl, hd), float("nan"), dtype=dev[0].dtype, device="cuda")
    uly.ulysses_seq_to_head(dev, rank, out)
    torch.cuda.synchronize()
    return out


CASES = [
    # P, n_local, bs, heads, hd, dtype
    (2, 128, 1, 4, 64, "f32"),      # the emulated P=2 rank share (fp32)
    (8, 64, 1, 32, 128, "bf16"),    # Llama-8B-shaped query heads
    (8, 64, 1, 8, 128, "bf16"),     # its key/value heads (one per rank)
    (8, 33, 2, 2, 128, "bf16"),     # replicated key/value heads, ragged n, batch 2
    (4, 5, 3, 8, 64, "bf16"),
    (1, 7, 1, 3, 64, "bf16"),       # P = 1: identity
    (3, 1, 1, 6, 32, "f32"),
]


@pytest.mark.parametrize("P,n,bs,heads,hd,dtype", CASES)
def test_seq_to_head_bit_exact_for_every_rank(P, n, bs, heads, hd, dtype):
    full = synth.normal(77, 1, (P * n, bs, heads, hd), dtype=dtype)
    chunks = [np.ascontiguousarray(full[c * n:(c + 1) * n]) for c in range(P)]
    for rank in range(P):
        got = run_seq_to_head(chunks, rank, dtype)
        want = oracle.seq_to_head(chunks, rank)
        assert storage_bytes(got) == want.tobytes(), f"rank {rank}"


@pytest.mark.parametrize("P,n,bs,heads,hd,dtype", [c for c in CASES if c[3] % c[0] == 0])
def test_head_to_seq_bit_exact_and_leaves_other_slots(P, n, bs, heads, hd, dtype):
    import torch
    import ulysses_sp_attention_amd as uly
    hl = heads // P
    canary = synth.normal(78, 2, (n, bs, heads, hd), dtype=dtype)
    for rank in range(P):
        x = synth.normal(79, 3 + rank, (P * n, bs, hl, hd), dtype=dtype)
        dev_chunks = [to_device(canary, dtype) for _ in range(P)]
        uly.ulysses_head_to_seq(to_device(x, dtype), rank, dev_chunks)
        torch.cuda.synchronize()
        want = [canary.copy() for _ in range(P)]
        oracle.head_to_seq(x, want, rank)
        for c in range(P):
            assert storage_bytes(dev_chunks[c]) == want[c].tobytes(), f"rank {rank} chunk {c}"


def test_empty_exchange_is_a_no_op():
    import torch
    import ulysses_sp_attention_amd as uly
    chunks = [torch.zeros((0, 1, 8, 128), dtype=torch.bfloat16, device="cuda") for _ in range(8)]
    # the empty head buffer is a zero-row view at the start of a sentinel row,
    # so that a stray write would show
    sentinel = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    out = sentinel[:0]
    uly.ulysses_seq_to_head(chunks, 3, out)
    uly.ulysses_head_to_seq(out, 3, chunks)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 0)


@pytest.mark.parametrize("name", ["llama8b-share-32k", "llama8b-share-128k"])
def test_full_size_pack_unpack_bit_exact(name):
    """Q, K, V packs and the O unpack at the benchmark's sizes (8 chunks)."""
    import torch
    import ulysses_sp_attention_amd as uly
    w = synth.WORKLOADS[name]
    n = w.n_local
    for stream, heads in ((synth.STREAM_Q, w.hq), (synth.STREAM_K, w.hkv), (synth.STREAM_V, w.hkv)):
        full = w.seq_tensor(stream, heads)
        dev_full = to_device(full, w.dtype)
        dev_chunks = [dev_full[c * n:(c + 1) * n] for c in range(w.P)]
        hl = heads // w.P
        out = torch.empty((w.seqlen, w.bs, hl, w.head_dim), dtype=torch.bfloat16, device="cuda")
        uly.ulysses_seq_to_head(dev_chunks, w.rank, out)
        torch.cuda.synchronize()
        want = oracle.seq_to_head([full[c * n:(c + 1) * n] for c in range(w.P)], w.rank)
        assert np.array_equal(host_storage(out), want), f"stream {stream}"
        del dev_full, dev_chunks
        if stream == synth.STREAM_Q:
            # unpack a head-sharded tensor back into the chunks' rank slots
            x = synth.normal(w.seed, 9, (w.seqlen, w.bs, hl, w.head_dim), dtype="bf16")
            canary = synth.normal(w.seed, 10, (n, w.bs, heads, w.head_dim), dtype="bf16")
            dev_chunks = [to_device(canary, "bf16") for _ in range(w.P)]
            uly.ulysses_head_to_seq(to_device(x, "bf16"), w.rank, dev_chunks)
            torch.cuda.synchronize()
            want_chunks = [canary.copy() for _ in range(w.P)]
            oracle.head_to_seq(x, want_chunks, w.rank)
            for c in range(w.P):
                assert np.array_equal(host_storage(dev_chunks[c]), want_chunks[c]), f"chunk {c}"
            del dev_chunks
        torch.cuda.empty_cache()


@pytest.mark.parametrize("P,n,bs,hd,heads_list,dtype", [
    (8, 64, 1, 128, (32, 8, 8), "bf16"),        # one layer's Q, K, V at the Llama-8B shape
    (8, 33, 2, 128, (32, 2, 2, 32), "bf16"),    # replicated key/value heads, ragged n, four tensors
    (2, 40, 1, 64, (4, 2), "f32"),
])
def test_batched_seq_to_head_matches_oracle_per_tensor(P, n, bs, hd, heads_list, dtype):
    import torch
    import ulysses_sp_attention_amd as uly
    fulls = [synth.normal(90 + i, 1, (P * n, bs, h, hd), dtype=dtype) for i, h in enumerate(heads_list)]
    chunk_sets = [[np.ascontiguousarray(f[c * n:(c + 1) * n]) for c in range(P)] for f in fulls]
    for rank in range(P):
        pairs = []
        for chunks, h in zip(chunk_sets, heads_list):
            dev = [to_device(c, dtype) for c in chunks]
            hl = h // P if h >= P else 1
            out = torch.full((P * n, bs, hl, hd), float("nan"), dtype=dev[0].dtype, device="cuda")
            pairs.append((dev, out))
        uly.ulysses_seq_to_head_batch(pairs, rank)
        torch.cuda.synchronize()
        for i, (chunks, (_, out)) in enumerate(zip(chunk_sets, pairs)):
            want = oracle.seq_to_head(chunks, rank)
            assert storage_bytes(out) == want.tobytes(), f"rank {rank} tensor {i}"


@pytest.mark.parametrize("P,n,bs,hd,heads_list,dtype", [
    (8, 64, 1, 128, (32, 8, 8), "bf16"),        # dQ, dK, dV of one layer
    (4, 17, 3, 64, (4, 8), "bf16"),
])
def test_batched_head_to_seq_matches_oracle_and_leaves_other_slots(P, n, bs, hd, heads_list, dtype):
    import torch
    import ulysses_sp_attention_amd as uly
    for rank in range(P):
        pairs, expect = [], []
        for i, h in enumerate(heads_list):
            hl = h // P
            canary = synth.normal(95 + i, 2, (n, bs, h, hd), dtype=dtype)
            x = synth.normal(96 + i, 3 + rank, (P * n, bs, hl, hd), dtype=dtype)
            dev_chunks = [to_device(canary, dtype) for _ in range(P)]
            pairs.append((to_device(x, dtype), dev_chunks))
            want = [canary.copy() for _ in range(P)]
            oracle.head_to_seq(x, want, rank)
            expect.append(want)
        uly.ulysses_head_to_seq_batch(pairs, rank)
        torch.cuda.synchronize()
        for i, ((_, dev_chunks), want) in enumerate(zip(pairs, expect)):
            for c in range(P):
                assert storage_bytes(dev_chunks[c]) == want[c].tobytes(), f"rank {rank} tensor {i} chunk {c}"
