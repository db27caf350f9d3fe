"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (so these
calls are safe without a device: no kernel is ever launched here)."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_library
import ulysses_sp_attention_amd as uly

HEADER = os.path.join(ROOT, "include", "ulysses.h")
FAKE = 0x10000          # 16-byte aligned stand-in device address, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    return ensure_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulysses_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(uly.EXPORTED_SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert uly.ulysses_abi_version() == uly.ABI_VERSION
    for code in range(9):
        s = uly.ulysses_status_string(code)
        assert s and s != "unknown status"
    assert uly.ulysses_status_string(1234) == "unknown status"


def chunk_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


@pytest.mark.parametrize("args,want", [
    # (chunks, P, rank, n_local, bs, heads, head_dim, dtype, out) -> status
    ((None, 2, 0, 4, 1, 4, 64, uly.FP32, FAKE), uly.ERR_NULL),
    (("ok", 2, 0, 4, 1, 4, 64, uly.FP32, None), uly.ERR_NULL),
    (("ok", 2, 0, 4, 1, 4, 64, 7, FAKE), uly.ERR_DTYPE),
    (("ok", 2, 2, 4, 1, 4, 64, uly.FP32, FAKE), uly.ERR_SHAPE),
    (("ok", 2, -1, 4, 1, 4, 64, uly.FP32, FAKE), uly.ERR_SHAPE),
    (("ok", 2, 0, -1, 1, 4, 64, uly.FP32, FAKE), uly.ERR_SHAPE),
    (("ok", 2, 0, 4, 0, 4, 64, uly.FP32, FAKE), uly.ERR_SHAPE),
    (("ok", 2, 0, 4, 1, 3, 64, uly.FP32, FAKE), uly.ERR_DIVISIBILITY),
    (("ok8", 8, 0, 4, 1, 12, 128, uly.BF16, FAKE), uly.ERR_DIVISIBILITY),
    (("ok8", 8, 0, 4, 1, 3, 128, uly.BF16, FAKE), uly.ERR_DIVISIBILITY),
    (("ok", 2, 0, 4, 1, 4, 4, uly.BF16, FAKE), uly.ERR_ALIGNMENT),
    (("ok", 2, 0, 4, 1, 4, 64, uly.FP32, MISALIGNED), uly.ERR_ALIGNMENT),
    (("bad", 2, 0, 4, 1, 4, 64, uly.FP32, FAKE), uly.ERR_ALIGNMENT),
    (("null", 2, 0, 4, 1, 4, 64, uly.FP32, FAKE), uly.ERR_NULL),
    (("ok", 2, 0, 0, 1, 4, 64, uly.FP32, FAKE), uly.OK),   # empty exchange: no launch
])
def test_seq_to_head_validation(lib, args, want):
    chunks, P, rank, n, bs, heads, hd, dt, out = args
    table = {"ok": [FAKE, FAKE + 4096], "ok8": [FAKE + 4096 * i for i in range(8)],
             "bad": [FAKE, MISALIGNED], "null": [FAKE, None]}
    arr = None if chunks is None else chunk_array(table[chunks])
    assert lib.ulysses_seq_to_head(arr, P, rank, n, bs, heads, hd, dt, out, None) == want


def test_head_to_seq_requires_heads_divisible_by_P(lib):
    arr = chunk_array([FAKE + 4096 * i for i in range(8)])
    # replicated key/value heads (heads < P) cannot be scattered back by one rank
    assert lib.ulysses_head_to_seq(FAKE, 8, 0, 4, 1, 2, 128, uly.BF16, arr, None) == uly.ERR_DIVISIBILITY
    assert lib.ulysses_head_to_seq(None, 8, 0, 4, 1, 8, 128, uly.BF16, arr, None) == uly.ERR_NULL
    assert lib.ulysses_head_to_seq(FAKE, 8, 0, 0, 1, 8, 128, uly.BF16, arr, None) == uly.OK


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, N=128, bs=1, hq=4, hkv=1, hd=128, dt=uly.BF16, scale=0.1,
             causal=1, cu=None, n_docs=0, o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.ulysses_attn_fwd(a["q"], a["k"], a["v"], a["N"], a["bs"], a["hq"], a["hkv"], a["hd"],
                                a["dt"], a["scale"], a["causal"], a["cu"], a["n_docs"], a["o"],
                                a["lse"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), uly.ERR_NULL), (dict(lse=None), uly.ERR_NULL),
    (dict(dt=5), uly.ERR_DTYPE),
    (dict(hd=96), uly.ERR_SHAPE), (dict(hd=256), uly.ERR_SHAPE),
    (dict(dt=uly.FP32, hd=48), uly.ERR_SHAPE),
    (dict(scale=0.0), uly.ERR_SHAPE), (dict(scale=-1.0), uly.ERR_SHAPE),
    (dict(scale=float("inf")), uly.ERR_SHAPE), (dict(scale=float("nan")), uly.ERR_SHAPE),
    (dict(N=-1), uly.ERR_SHAPE), (dict(bs=0), uly.ERR_SHAPE),
    (dict(hq=6, hkv=4), uly.ERR_DIVISIBILITY),
    (dict(cu=FAKE, n_docs=2, bs=2), uly.ERR_SHAPE),
    (dict(cu=FAKE, n_docs=0), uly.ERR_SHAPE),
    (dict(cu=FAKE, n_docs=129), uly.ERR_SHAPE),
    (dict(cu=FAKE + 2, n_docs=2), uly.ERR_ALIGNMENT),
    (dict(q=MISALIGNED), uly.ERR_ALIGNMENT), (dict(o=MISALIGNED), uly.ERR_ALIGNMENT),
    (dict(lse=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(N=0), uly.OK),
    # sizes the kernels count in 32 bits
    (dict(N=1 << 30), uly.ERR_UNSUPPORTED),
    (dict(N=1 << 29, hq=1024, hkv=1), uly.ERR_UNSUPPORTED),
    (dict(bs=256, hq=256, hkv=256), uly.ERR_UNSUPPORTED),
])
def test_attn_fwd_validation(lib, kw, want):
    assert fwd(lib, **kw) == want


def merge(lib, **kw):
    a = dict(oa=FAKE, la=FAKE, ob=FAKE, lb=FAKE, N=128, bs=1, heads=4, hd=128, dt=uly.BF16,
             o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.ulysses_attn_merge(a["oa"], a["la"], a["ob"], a["lb"], a["N"], a["bs"], a["heads"],
                                  a["hd"], a["dt"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(oa=None), uly.ERR_NULL), (dict(lb=None), uly.ERR_NULL), (dict(o=None), uly.ERR_NULL),
    (dict(lse=None), uly.ERR_NULL),
    (dict(dt=7), uly.ERR_DTYPE),
    (dict(hd=96), uly.ERR_SHAPE), (dict(hd=256), uly.ERR_SHAPE), (dict(hd=16), uly.ERR_SHAPE),
    (dict(N=-1), uly.ERR_SHAPE), (dict(bs=0), uly.ERR_SHAPE), (dict(heads=0), uly.ERR_SHAPE),
    (dict(N=1 << 30), uly.ERR_UNSUPPORTED), (dict(bs=256, heads=256), uly.ERR_UNSUPPORTED),
    (dict(oa=MISALIGNED), uly.ERR_ALIGNMENT), (dict(ob=MISALIGNED), uly.ERR_ALIGNMENT),
    (dict(o=MISALIGNED), uly.ERR_ALIGNMENT), (dict(la=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(lse=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(N=0), uly.OK), (dict(dt=uly.FP32, hd=32, N=0), uly.OK),
])
def test_attn_merge_validation(lib, kw, want):
    assert merge(lib, **kw) == want


def test_attn_bwd_workspace_rules(lib):
    need = lib.ulysses_attn_bwd_workspace_size(1000, 2, 4, 1, 128, uly.BF16)
    assert need >= 1000 * 2 * 4 * 4 and need % 256 == 0
    assert lib.ulysses_attn_bwd_workspace_size(1000, 2, 4, 3, 128, uly.BF16) == 0   # invalid shape
    common = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1000, 2, 4, 1, 128, uly.BF16, 0.1, 1, None, 0,
              FAKE, FAKE, FAKE)
    assert lib.ulysses_attn_bwd(*common, None, need, None) == uly.ERR_WORKSPACE
    assert lib.ulysses_attn_bwd(*common, FAKE, need - 1, None) == uly.ERR_WORKSPACE
    bad = list(common)
    bad[5] = None   # dout
    assert lib.ulysses_attn_bwd(*bad, FAKE, need, None) == uly.ERR_NULL
    bad = list(common)
    bad[16] = MISALIGNED   # dq
    assert lib.ulysses_attn_bwd(*bad, FAKE, need, None) == uly.ERR_ALIGNMENT


def test_binding_raises_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(uly, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        uly.load_library(str(tmp_path / "missing.so"))


def batch_descs(specs):
    """specs: [(chunk table key or None, head pointer, heads)] -> ctypes array + keep-alive."""
    table = {"ok": [FAKE, FAKE + 4096], "ok8": [FAKE + 4096 * i for i in range(8)],
             "bad": [FAKE, MISALIGNED], "null": [FAKE, None]}
    descs = (uly.ExchangeTensor * max(1, len(specs)))()
    keep = []
    for i, (key, head, heads) in enumerate(specs):
        arr = None if key is None else chunk_array(table[key])
        keep.append(arr)
        descs[i].chunks = None if arr is None else ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        descs[i].head = head
        descs[i].heads = heads
    return descs, keep


@pytest.mark.parametrize("specs,n,n_local,want", [
    # every failing case is rejected before any launch
    ([("ok", FAKE, 4)], 0, 4, uly.ERR_SHAPE),
    ([("ok", FAKE, 4)] * 4, 5, 4, uly.ERR_SHAPE),
    ([("ok", FAKE, 4), ("ok", FAKE + 65536, 3)], 2, 4, uly.ERR_DIVISIBILITY),
    ([("ok", FAKE, 4), (None, FAKE + 65536, 4)], 2, 4, uly.ERR_NULL),
    ([("ok", FAKE, 4), ("null", FAKE + 65536, 4)], 2, 4, uly.ERR_NULL),
    ([("ok", FAKE, 4), ("ok", MISALIGNED, 4)], 2, 4, uly.ERR_ALIGNMENT),
    ([("bad", FAKE, 4), ("ok", FAKE + 65536, 4)], 2, 4, uly.ERR_ALIGNMENT),
    ([("ok", FAKE, 4), ("ok", None, 4)], 2, 4, uly.ERR_NULL),
    ([("ok", FAKE, 4), ("ok", FAKE + 65536, 2)], 2, 0, uly.OK),   # empty: no launch
])
def test_batch_exchange_validation(lib, specs, n, n_local, want):
    descs, keep = batch_descs(specs)
    for fn in (lib.ulysses_seq_to_head_batch, lib.ulysses_head_to_seq_batch):
        assert fn(descs, n, 2, 0, n_local, 1, 64, uly.FP32, None) == want


def test_batch_exchange_null_table_and_head_to_seq_divisibility(lib):
    assert lib.ulysses_seq_to_head_batch(None, 1, 2, 0, 4, 1, 64, uly.FP32, None) == uly.ERR_NULL
    # replicated key/value heads (heads < P) are fine for seq_to_head, not for head_to_seq
    descs, keep = batch_descs([("ok8", FAKE, 8), ("ok8", FAKE + 65536, 2)])
    assert lib.ulysses_head_to_seq_batch(descs, 2, 8, 0, 4, 1, 128, uly.BF16, None) == \
        uly.ERR_DIVISIBILITY


def fused_fwd(lib, P=4, table=None, o_table=None, **kw):
    a = dict(rank=1, n=128, bs=1, hq=8, hkv=4, hd=128, dt=uly.BF16, scale=0.1, causal=1, cu=None,
             n_docs=0, lse=FAKE)
    a.update(kw)
    t = chunk_array(table if table is not None else [FAKE + 4096 * i for i in range(P)])
    ot = chunk_array(o_table if o_table is not None else [FAKE + 4096 * i for i in range(P)])
    return lib.ulysses_attn_fwd_fused(t, t, t, P, a["rank"], a["n"], a["bs"], a["hq"], a["hkv"],
                                      a["hd"], a["dt"], a["scale"], a["causal"], a["cu"],
                                      a["n_docs"], ot, a["lse"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(lse=None), uly.ERR_NULL),
    (dict(table=[FAKE, None, FAKE, FAKE]), uly.ERR_NULL),
    (dict(o_table=[FAKE, FAKE, FAKE, None]), uly.ERR_NULL),
    (dict(table=[FAKE, MISALIGNED, FAKE, FAKE]), uly.ERR_ALIGNMENT),
    (dict(lse=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(rank=4), uly.ERR_SHAPE), (dict(rank=-1), uly.ERR_SHAPE), (dict(n=-64), uly.ERR_SHAPE),
    (dict(hq=6), uly.ERR_DIVISIBILITY),              # q heads not divisible by P
    (dict(hkv=3), uly.ERR_DIVISIBILITY),             # kv heads neither multiple nor divisor of P
    (dict(hd=96), uly.ERR_SHAPE), (dict(dt=9), uly.ERR_DTYPE),
    (dict(dt=uly.FP32), uly.ERR_UNSUPPORTED),       # bf16 kernels only
    (dict(n=100), uly.ERR_UNSUPPORTED),             # 64-row tiles must not straddle chunks
    (dict(bs=128, hq=1024, hkv=4), uly.ERR_UNSUPPORTED),   # 64 rows of all heads beyond 2^31 bytes
    (dict(n=0), uly.OK),
    (dict(n=0, hkv=2), uly.OK),                     # replicated kv heads accepted
])
def test_attn_fwd_fused_validation(lib, kw, want):
    assert fused_fwd(lib, **kw) == want


def test_attn_fwd_fused_rejects_more_than_16_chunks(lib):
    table = [FAKE + 4096 * i for i in range(17)]
    assert fused_fwd(lib, P=17, table=table, o_table=table, hq=34, hkv=17, rank=0) == \
        uly.ERR_UNSUPPORTED


def fused_bwd(lib, P=4, table=None, out_table=None, ws_bytes=None, **kw):
    a = dict(rank=1, n=128, bs=1, hq=8, hkv=4, hd=128, dt=uly.BF16, scale=0.1, causal=1, cu=None,
             n_docs=0, lse=FAKE, ws=FAKE)
    a.update(kw)
    t = chunk_array(table if table is not None else [FAKE + 4096 * i for i in range(P)])
    ot = chunk_array(out_table if out_table is not None else [FAKE + 4096 * i for i in range(P)])
    if ws_bytes is None:
        hkv_l = a["hkv"] // P if a["hkv"] >= P else 1
        ws_bytes = max(lib.ulysses_attn_bwd_workspace_size(P * a["n"], a["bs"], a["hq"] // P,
                                                           hkv_l, a["hd"], uly.BF16), 1)
    return lib.ulysses_attn_bwd_fused(t, t, t, t, a["lse"], t, P, a["rank"], a["n"], a["bs"],
                                      a["hq"], a["hkv"], a["hd"], a["dt"], a["scale"], a["causal"],
                                      a["cu"], a["n_docs"], ot, ot, ot, a["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(lse=None), uly.ERR_NULL),
    (dict(table=[FAKE, None, FAKE, FAKE]), uly.ERR_NULL),
    (dict(out_table=[FAKE, FAKE, None, FAKE]), uly.ERR_NULL),
    (dict(table=[FAKE, FAKE, MISALIGNED, FAKE]), uly.ERR_ALIGNMENT),
    (dict(out_table=[MISALIGNED, FAKE, FAKE, FAKE]), uly.ERR_ALIGNMENT),
    (dict(lse=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(ws=None), uly.ERR_WORKSPACE),
    (dict(ws_bytes=8191), uly.ERR_WORKSPACE),         # needs 2 * 512 rows * 2 heads * 4 bytes
    (dict(ws=FAKE + 8), uly.ERR_ALIGNMENT),
    (dict(rank=4), uly.ERR_SHAPE), (dict(n=-64), uly.ERR_SHAPE),
    (dict(hq=6), uly.ERR_DIVISIBILITY),
    (dict(hkv=2), uly.ERR_DIVISIBILITY),               # replicated kv heads: dK/dV need a sum
    (dict(hkv=2, n=0), uly.ERR_DIVISIBILITY),
    (dict(hd=96), uly.ERR_SHAPE), (dict(dt=9), uly.ERR_DTYPE),
    (dict(dt=uly.FP32), uly.ERR_UNSUPPORTED),
    (dict(n=100), uly.ERR_UNSUPPORTED),
    (dict(n=0, ws=None), uly.OK),                      # empty: no workspace needed
])
def test_attn_bwd_fused_validation(lib, kw, want):
    assert fused_bwd(lib, **kw) == want


def logits_loss_call(lib, **kw):
    a = dict(h=FAKE, w=FAKE, labels=FAKE, T=64, d=128, V=1000, dt=uly.BF16, ignore=-100,
             s=1.0, shard=32, rows=FAKE, total=FAKE, good=FAKE, dh=FAKE, dw=FAKE, ws=FAKE,
             ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = max(lib.ulysses_logits_loss_workspace_size(min(a["shard"], max(a["T"], 1)),
                                                                   a["V"]), 1)
    return lib.ulysses_logits_loss(a["h"], a["w"], a["labels"], a["T"], a["d"], a["V"], a["dt"],
                                   a["ignore"], a["s"], a["shard"], a["rows"], a["total"],
                                   a["good"], a["dh"], a["dw"], a["ws"], a["ws_bytes"], None)


def test_logits_loss_workspace_size(lib):
    # bf16 exp(Z - m) / G of one shard with rows padded to 8 columns, the
    # (max, sum) pair of every row and 256-column tile, and one fp32 label
    # logit per row, each region rounded up to 256 bytes
    assert lib.ulysses_logits_loss_workspace_size(32, 1000) == 64000 + 1024 + 256
    assert lib.ulysses_logits_loss_workspace_size(3, 5) == 256 + 256 + 256
    assert lib.ulysses_logits_loss_workspace_size(2, 300) == 256 * 5 + 256 + 256
    assert lib.ulysses_logits_loss_workspace_size(0, 5) == 0
    assert lib.ulysses_logits_loss_workspace_size(4, 1 << 31) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(w=None), uly.ERR_NULL), (dict(h=None), uly.ERR_NULL), (dict(labels=None), uly.ERR_NULL),
    (dict(dw=None), uly.ERR_NULL), (dict(total=None), uly.ERR_NULL), (dict(dh=None), uly.ERR_NULL),
    (dict(dt=9), uly.ERR_DTYPE),
    (dict(dt=uly.FP32), uly.ERR_UNSUPPORTED),
    (dict(T=-1), uly.ERR_SHAPE), (dict(d=0), uly.ERR_SHAPE), (dict(V=0), uly.ERR_SHAPE),
    (dict(d=12), uly.ERR_SHAPE),
    (dict(shard=0), uly.ERR_SHAPE), (dict(s=float("nan")), uly.ERR_SHAPE),
    (dict(s=float("inf")), uly.ERR_SHAPE),
    (dict(V=1 << 31), uly.ERR_UNSUPPORTED), (dict(d=1 << 31), uly.ERR_UNSUPPORTED),
    (dict(h=MISALIGNED), uly.ERR_ALIGNMENT), (dict(dw=MISALIGNED), uly.ERR_ALIGNMENT),
    (dict(labels=FAKE + 4), uly.ERR_ALIGNMENT), (dict(good=FAKE + 4), uly.ERR_ALIGNMENT),
    (dict(rows=FAKE + 2), uly.ERR_ALIGNMENT),
    (dict(ws=None), uly.ERR_WORKSPACE),
    (dict(ws_bytes=64000 + 1024 + 256 - 1), uly.ERR_WORKSPACE),
    (dict(ws=FAKE + 8), uly.ERR_ALIGNMENT),
])
def test_logits_loss_validation(lib, kw, want):
    assert logits_loss_call(lib, **kw) == want


def mlp_call(lib, backward, **kw):
    a = dict(x=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, dy=FAKE, T=64, d=128, I=256, dt=uly.BF16,
             shard=32, y=FAKE, dx=FAKE, dwg=FAKE, dwu=FAKE, dwd=FAKE, ws=FAKE, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = max(lib.ulysses_tiled_mlp_workspace_size(
            min(a["shard"], max(a["T"], 1)), max(a["d"], 1), max(a["I"], 1), int(backward)), 1)
    if backward:
        return lib.ulysses_tiled_mlp_bwd(a["x"], a["wg"], a["wu"], a["wd"], a["dy"], a["T"], a["d"],
                                         a["I"], a["dt"], a["shard"], a["dx"], a["dwg"], a["dwu"],
                                         a["dwd"], a["ws"], a["ws_bytes"], None)
    return lib.ulysses_tiled_mlp_fwd(a["x"], a["wg"], a["wu"], a["wd"], a["T"], a["d"], a["I"],
                                     a["dt"], a["shard"], a["y"], a["ws"], a["ws_bytes"], None)


def test_tiled_mlp_workspace_size(lib):
    S, d, inter = 32, 128, 256
    f, h = S * inter * 4, S * inter * 2      # multiples of 256 here
    assert lib.ulysses_tiled_mlp_workspace_size(S, d, inter, 0) == 2 * f + h
    assert lib.ulysses_tiled_mlp_workspace_size(S, d, inter, 1) == 3 * f + 3 * h + S * d * 4
    assert lib.ulysses_tiled_mlp_workspace_size(0, d, inter, 1) == 0


@pytest.mark.parametrize("backward", [False, True])
@pytest.mark.parametrize("kw,want", [
    (dict(wg=None), uly.ERR_NULL), (dict(wd=None), uly.ERR_NULL), (dict(x=None), uly.ERR_NULL),
    (dict(dt=9), uly.ERR_DTYPE), (dict(dt=uly.FP32), uly.ERR_UNSUPPORTED),
    (dict(T=-1), uly.ERR_SHAPE), (dict(d=0), uly.ERR_SHAPE), (dict(I=0), uly.ERR_SHAPE),
    (dict(d=100), uly.ERR_SHAPE), (dict(I=36), uly.ERR_SHAPE),    # not multiples of 8
    (dict(shard=0), uly.ERR_SHAPE),
    (dict(I=1 << 31), uly.ERR_UNSUPPORTED),
    (dict(x=MISALIGNED), uly.ERR_ALIGNMENT), (dict(wu=MISALIGNED), uly.ERR_ALIGNMENT),
    (dict(ws=None), uly.ERR_WORKSPACE), (dict(ws_bytes=1), uly.ERR_WORKSPACE),
    (dict(ws=FAKE + 8), uly.ERR_ALIGNMENT),
])
def test_tiled_mlp_validation(lib, backward, kw, want):
    assert mlp_call(lib, backward, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(dy=None), uly.ERR_NULL), (dict(dx=None), uly.ERR_NULL), (dict(dwd=None), uly.ERR_NULL),
    (dict(dwg=MISALIGNED), uly.ERR_ALIGNMENT), (dict(dy=MISALIGNED), uly.ERR_ALIGNMENT),
])
def test_tiled_mlp_bwd_validation(lib, kw, want):
    assert mlp_call(lib, True, **kw) == want


def test_tiled_mlp_fwd_empty_is_a_no_op(lib):
    assert mlp_call(lib, False, T=0, x=None, y=None, ws=None) == uly.OK


def test_attn_bwd_noalloc_validation(lib):
    """The entry point without a workspace checks like ulysses_attn_bwd and
    refuses sizes whose statistics exceed its fixed scratch, before any HIP
    call; an empty sequence is a no-op that never looks the scratch up."""
    limit_rows = uly.NOALLOC_SCRATCH_BYTES // 8   # bf16: 2 fp32 statistics per row

    def call(N, hq=4, hkv=1, dtype=uly.BF16, ptr=FAKE, hd=128):
        return lib.ulysses_attn_bwd_noalloc(ptr, FAKE, FAKE, FAKE, FAKE, FAKE, N, 1, hq, hkv, hd,
                                            dtype, 0.088, 1, None, 0, FAKE, FAKE, FAKE, None)
    assert call(limit_rows // 4 + 64) == uly.ERR_WORKSPACE
    assert call(2 * limit_rows // 4 + 64, dtype=uly.FP32) == uly.ERR_WORKSPACE   # one statistic
    assert call(64, ptr=None) == uly.ERR_NULL
    assert call(64, ptr=MISALIGNED) == uly.ERR_ALIGNMENT
    assert call(64, hq=6, hkv=4) == uly.ERR_DIVISIBILITY
    assert call(0) == uly.OK
