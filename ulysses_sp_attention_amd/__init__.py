"""Python binding of libulysses (one rank's share of an Ulysses attention layer
on AMD Instinct MI355X).

Thin ctypes marshalling over the C-ABI declared in ``include/ulysses.h``:
each function below has the name of the C entry point it calls, takes torch
device tensors, passes their data pointers, sizes and the current HIP stream,
and raises :class:`UlyssesError` when the library returns a non-OK status.
Before any call it checks every tensor argument -- on the current GPU,
contiguous, of exactly the shape the entry point reads or writes and of a
consistent element type -- and raises ``ValueError`` otherwise, because the
library sees only pointers and sizes: a view, an undersized buffer or a host
tensor would make its kernels access memory they do not own.
All computation happens in the library's HIP kernels; torch only supplies
device memory and the stream.  The library must have been built
(``ulysses_sp_attention_amd._build.build_lib()``); importing the binding
without it raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# ULYSSES_LIB loads another build of the same library instead (the
# host-sanitizer build that tests/test_sanitizers.py makes); nothing else
# sets it.
LIB_PATH = os.environ.get("ULYSSES_LIB") or os.path.join(_PKG, "libulysses.so")

OK, ERR_NULL, ERR_SHAPE, ERR_DIVISIBILITY, ERR_DTYPE, ERR_ALIGNMENT, ERR_UNSUPPORTED, \
    ERR_WORKSPACE, ERR_HIP = range(9)
BF16, FP32 = 0, 1
ABI_VERSION = 7   # ULYSSES_ABI_VERSION this binding is written for
_INVALID_DTYPE = 99

# Every symbol include/ulysses.h declares.
EXPORTED_SYMBOLS = (
    "ulysses_abi_version", "ulysses_status_string", "ulysses_seq_to_head", "ulysses_head_to_seq",
    "ulysses_seq_to_head_batch", "ulysses_head_to_seq_batch",
    "ulysses_attn_fwd", "ulysses_attn_bwd_workspace_size", "ulysses_attn_bwd",
    "ulysses_attn_bwd_noalloc",
    "ulysses_attn_merge", "ulysses_attn_fwd_fused", "ulysses_attn_bwd_fused",
    "ulysses_logits_loss_workspace_size", "ulysses_logits_loss",
    "ulysses_tiled_mlp_workspace_size", "ulysses_tiled_mlp_fwd", "ulysses_tiled_mlp_bwd",
)
MAX_BATCH = 4   # ULYSSES_MAX_BATCH
NOALLOC_SCRATCH_BYTES = 16 << 20   # ULYSSES_NOALLOC_SCRATCH_BYTES


class ExchangeTensor(ctypes.Structure):
    """ulysses_exchange_tensor_t: P chunk pointers, the head buffer, global heads."""
    _fields_ = [("chunks", ctypes.POINTER(ctypes.c_void_p)), ("head", ctypes.c_void_p),
                ("heads", ctypes.c_int)]


class UlyssesError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: {message} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libulysses.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime (soname libamdhip64.so.7) and loads it
    # by an unversioned name.  Importing torch first makes the library's
    # dependency resolve to that same runtime, so tensors, streams and
    # kernels live in one HIP instance; loading libulysses first would bring
    # in a second runtime beside torch's.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"libulysses is not built ({path} missing); run "
                           "ulysses_sp_attention_amd._build.build_lib()")
    lib = ctypes.CDLL(path)
    vp, ci, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.ulysses_abi_version.argtypes = []
    lib.ulysses_abi_version.restype = ci
    lib.ulysses_status_string.argtypes = [ci]
    lib.ulysses_status_string.restype = ctypes.c_char_p
    lib.ulysses_seq_to_head.argtypes = [vp, ci, ci, i64, ci, ci, ci, ci, vp, vp]
    lib.ulysses_seq_to_head.restype = ci
    lib.ulysses_head_to_seq.argtypes = [vp, ci, ci, i64, ci, ci, ci, ci, vp, vp]
    lib.ulysses_head_to_seq.restype = ci
    for name in ("ulysses_seq_to_head_batch", "ulysses_head_to_seq_batch"):
        getattr(lib, name).argtypes = [ctypes.POINTER(ExchangeTensor), ci, ci, ci, i64, ci, ci, ci, vp]
        getattr(lib, name).restype = ci
    lib.ulysses_attn_fwd.argtypes = [vp, vp, vp, i64, ci, ci, ci, ci, ci, f32, ci, vp, ci, vp, vp, vp]
    lib.ulysses_attn_fwd.restype = ci
    lib.ulysses_attn_bwd_workspace_size.argtypes = [i64, ci, ci, ci, ci, ci]
    lib.ulysses_attn_bwd_workspace_size.restype = sz
    lib.ulysses_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, ci, ci, ci, ci, ci, f32, ci, vp, ci,
                                     vp, vp, vp, vp, sz, vp]
    lib.ulysses_attn_bwd.restype = ci
    lib.ulysses_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, ci, ci, ci, ci, ci, f32, ci,
                                             vp, ci, vp, vp, vp, vp]
    lib.ulysses_attn_bwd_noalloc.restype = ci
    lib.ulysses_attn_merge.argtypes = [vp, vp, vp, vp, i64, ci, ci, ci, ci, vp, vp, vp]
    lib.ulysses_attn_merge.restype = ci
    lib.ulysses_attn_fwd_fused.argtypes = [vp, vp, vp, ci, ci, i64, ci, ci, ci, ci, ci, f32, ci, vp,
                                           ci, vp, vp, vp]
    lib.ulysses_attn_fwd_fused.restype = ci
    lib.ulysses_attn_bwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, i64, ci, ci, ci, ci, ci,
                                           f32, ci, vp, ci, vp, vp, vp, vp, sz, vp]
    lib.ulysses_attn_bwd_fused.restype = ci
    lib.ulysses_logits_loss_workspace_size.argtypes = [i64, i64]
    lib.ulysses_logits_loss_workspace_size.restype = sz
    lib.ulysses_logits_loss.argtypes = [vp, vp, vp, i64, i64, i64, ci, i64, f32, i64, vp, vp, vp, vp,
                                        vp, vp, sz, vp]
    lib.ulysses_logits_loss.restype = ci
    lib.ulysses_tiled_mlp_workspace_size.argtypes = [i64, i64, i64, ci]
    lib.ulysses_tiled_mlp_workspace_size.restype = sz
    lib.ulysses_tiled_mlp_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, i64, vp, vp, sz, vp]
    lib.ulysses_tiled_mlp_fwd.restype = ci
    lib.ulysses_tiled_mlp_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, i64, vp, vp, vp,
                                          vp, vp, sz, vp]
    lib.ulysses_tiled_mlp_bwd.restype = ci
    _lib = lib
    return lib


def _check(func: str, status: int) -> None:
    if status != OK:
        raise UlyssesError(func, status, ulysses_status_string(status))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    return _INVALID_DTYPE   # the library reports ERR_DTYPE


def _ptr(t):
    return None if t is None else t.data_ptr()


def _device_ok(t) -> bool:
    """t lives on the GPU the library launches on (the current device)."""
    import torch
    return t.device.type == "cuda" and t.device.index == torch.cuda.current_device()


def _need(name: str, t, shape, dtype=None) -> None:
    """Raise ValueError unless t is a contiguous tensor on the current GPU with
    exactly `shape` (and element type `dtype`, when given)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not _device_ok(t):
        raise ValueError(f"{name}: must be on the current GPU (got {t.device})")


def _need_4d(name: str, t) -> tuple:
    """A contiguous [seq, bs, heads, head_dim] GPU tensor; returns its shape."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() != 4:
        raise ValueError(f"{name}: expected a 4-D [seq, bs, heads, head_dim] tensor")
    _need(name, t, t.shape)
    return tuple(t.shape)


def _need_chunks(name: str, chunks, heads=None, dtype=None) -> tuple:
    """P alike contiguous chunks [n_local, bs, heads, head_dim]; returns
    (P, n_local, bs, heads, head_dim)."""
    if not isinstance(chunks, (list, tuple)) or len(chunks) == 0:
        raise ValueError(f"{name}: expected a non-empty list of chunk tensors")
    n, bs, h, hd = _need_4d(f"{name}[0]", chunks[0])
    if heads is not None and h != heads:
        raise ValueError(f"{name}: {h} heads per chunk, expected {heads}")
    dt = chunks[0].dtype if dtype is None else dtype
    for i, c in enumerate(chunks):
        _need(f"{name}[{i}]", c, (n, bs, h, hd), dt)
    return len(chunks), n, bs, h, hd


def _need_workspace(t) -> None:
    if t is None:
        return   # the library reports ERR_NULL / ERR_WORKSPACE
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("workspace: expected a torch tensor")
    _need("workspace", t, t.shape)


def _need_cu(cu_seqlens) -> None:
    if cu_seqlens is None:
        return
    import torch
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens: expected a 1-D tensor of n_docs + 1 >= 2 offsets")
    _need("cu_seqlens", cu_seqlens, cu_seqlens.shape, torch.int32)


def _local_heads(heads: int, P: int) -> int:
    return heads // P if heads >= P else 1


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def ulysses_abi_version() -> int:
    return int(load_library().ulysses_abi_version())


def ulysses_status_string(status: int) -> str:
    return load_library().ulysses_status_string(status).decode()


def ulysses_seq_to_head(chunks, rank: int, out, stream=None) -> None:
    """chunks: P tensors [n_local, bs, heads, head_dim]; out: [P*n_local, bs, heads_l, head_dim]."""
    P, n, bs, heads, hd = _need_chunks("chunks", chunks)
    _need("out", out, (P * n, bs, _local_heads(heads, P), hd), chunks[0].dtype)
    st = load_library().ulysses_seq_to_head(
        _ptr_array(chunks), len(chunks), rank, n, bs, heads, hd, _dtype_code(chunks[0]), _ptr(out),
        _stream(stream))
    _check("ulysses_seq_to_head", st)


def ulysses_head_to_seq(inp, rank: int, chunks, stream=None) -> None:
    """inp: [P*n_local, bs, heads/P, head_dim]; writes rank's head slots of the P chunks."""
    P, n, bs, heads, hd = _need_chunks("chunks", chunks)
    _need("inp", inp, (P * n, bs, heads // P, hd), chunks[0].dtype)
    st = load_library().ulysses_head_to_seq(
        _ptr(inp), len(chunks), rank, n, bs, heads, hd, _dtype_code(inp), _ptr_array(chunks),
        _stream(stream))
    _check("ulysses_head_to_seq", st)


def _batch_descs(pairs):
    """[(chunks, head_tensor)] -> ctypes array of ExchangeTensor (+ keep-alive list)."""
    if not isinstance(pairs, (list, tuple)) or not pairs:
        raise ValueError("batched exchange: expected a non-empty list of (chunks, head) pairs")
    P, n, bs, _, hd = _need_chunks("pairs[0] chunks", pairs[0][0])
    for i, (chunks, head) in enumerate(pairs):
        Pi, ni, bsi, hi, hdi = _need_chunks(f"pairs[{i}] chunks", chunks, dtype=pairs[0][0][0].dtype)
        if (Pi, ni, bsi, hdi) != (P, n, bs, hd):
            raise ValueError("batched exchange: tensors differ in P, n_local, bs or head_dim")
        _need(f"pairs[{i}] head", head, (P * n, bs, _local_heads(hi, P), hd), chunks[0].dtype)
    descs = (ExchangeTensor * len(pairs))()
    keep = []
    for i, (chunks, head) in enumerate(pairs):
        arr = _ptr_array(chunks)
        keep.append(arr)
        descs[i].chunks = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        descs[i].head = head.data_ptr()
        descs[i].heads = chunks[0].shape[2]
    return descs, keep


def ulysses_seq_to_head_batch(pairs, rank: int, stream=None) -> None:
    """pairs: up to MAX_BATCH (chunks, out) as for ulysses_seq_to_head, moved in one launch.
    All tensors share P, n_local, bs, head_dim and dtype; head counts may differ."""
    descs, keep = _batch_descs(pairs)
    n, bs, _, hd = pairs[0][0][0].shape
    st = load_library().ulysses_seq_to_head_batch(
        descs, len(pairs), len(pairs[0][0]), rank, n, bs, hd, _dtype_code(pairs[0][0][0]),
        _stream(stream))
    del keep
    _check("ulysses_seq_to_head_batch", st)


def ulysses_head_to_seq_batch(pairs, rank: int, stream=None) -> None:
    """pairs: up to MAX_BATCH (inp, chunks) as for ulysses_head_to_seq, moved in one launch."""
    if not isinstance(pairs, (list, tuple)) or not pairs:
        raise ValueError("batched exchange: expected a non-empty list of (inp, chunks) pairs")
    descs, keep = _batch_descs([(chunks, inp) for inp, chunks in pairs])
    n, bs, _, hd = pairs[0][1][0].shape
    st = load_library().ulysses_head_to_seq_batch(
        descs, len(pairs), len(pairs[0][1]), rank, n, bs, hd, _dtype_code(pairs[0][0]),
        _stream(stream))
    del keep
    _check("ulysses_head_to_seq_batch", st)


def ulysses_attn_fwd(q, k, v, o, lse, softmax_scale: float, causal: bool = True,
                     cu_seqlens=None, stream=None) -> None:
    """q, o: [N, bs, hq, hd]; k, v: [N, bs, hkv, hd]; lse: fp32 [bs, hq, N];
    cu_seqlens: optional device int32 [n_docs + 1]."""
    import torch
    N, bs, hq, hd = _need_4d("q", q)
    hkv = _need_4d("k", k)[2]
    _need("k", k, (N, bs, hkv, hd), q.dtype)
    _need("v", v, (N, bs, hkv, hd), q.dtype)
    _need("o", o, (N, bs, hq, hd), q.dtype)
    _need("lse", lse, (bs, hq, N), torch.float32)
    _need_cu(cu_seqlens)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    st = load_library().ulysses_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), N, bs, hq, hkv, hd, _dtype_code(q), softmax_scale, int(causal),
        _ptr(cu_seqlens), n_docs, _ptr(o), _ptr(lse), _stream(stream))
    _check("ulysses_attn_fwd", st)


def ulysses_attn_bwd_workspace_size(seqlen: int, bs: int, hq: int, hkv: int, head_dim: int,
                                    dtype: int) -> int:
    return int(load_library().ulysses_attn_bwd_workspace_size(seqlen, bs, hq, hkv, head_dim, dtype))


def ulysses_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, softmax_scale: float,
                     causal: bool = True, cu_seqlens=None, stream=None) -> None:
    """Gradients of ulysses_attn_fwd.  workspace: device tensor of at least
    ulysses_attn_bwd_workspace_size(...) bytes."""
    import torch
    N, bs, hq, hd = _need_4d("q", q)
    hkv = _need_4d("k", k)[2]
    for name, t, h in (("k", k, hkv), ("v", v, hkv), ("o", o, hq), ("dout", dout, hq),
                       ("dq", dq, hq), ("dk", dk, hkv), ("dv", dv, hkv)):
        _need(name, t, (N, bs, h, hd), q.dtype)
    _need("lse", lse, (bs, hq, N), torch.float32)
    _need_cu(cu_seqlens)
    _need_workspace(workspace)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().ulysses_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), N, bs, hq, hkv, hd,
        _dtype_code(q), softmax_scale, int(causal), _ptr(cu_seqlens), n_docs, _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream))
    _check("ulysses_attn_bwd", st)


def ulysses_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, softmax_scale: float,
                             causal: bool = True, cu_seqlens=None, stream=None) -> None:
    """ulysses_attn_bwd without a workspace: the statistics go to the
    library's fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES), so the call
    allocates nothing.  Calls overlapping in time on one GPU race."""
    import torch
    N, bs, hq, hd = _need_4d("q", q)
    hkv = _need_4d("k", k)[2]
    for name, t, h in (("k", k, hkv), ("v", v, hkv), ("o", o, hq), ("dout", dout, hq),
                       ("dq", dq, hq), ("dk", dk, hkv), ("dv", dv, hkv)):
        _need(name, t, (N, bs, h, hd), q.dtype)
    _need("lse", lse, (bs, hq, N), torch.float32)
    _need_cu(cu_seqlens)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    st = load_library().ulysses_attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), N, bs, hq, hkv, hd,
        _dtype_code(q), softmax_scale, int(causal), _ptr(cu_seqlens), n_docs, _ptr(dq), _ptr(dk),
        _ptr(dv), _stream(stream))
    _check("ulysses_attn_bwd_noalloc", st)


def ulysses_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, stream=None) -> None:
    """Merge of two partial attention results over disjoint key sets.
    o_a, o_b, o: [N, bs, heads, hd]; lse_a, lse_b, lse: fp32 [bs, heads, N].
    o may be o_a or o_b and lse may be lse_a or lse_b (in place)."""
    import torch
    N, bs, heads, hd = _need_4d("o_a", o_a)
    _need("o_b", o_b, (N, bs, heads, hd), o_a.dtype)
    _need("o", o, (N, bs, heads, hd), o_a.dtype)
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b), ("lse", lse)):
        _need(name, t, (bs, heads, N), torch.float32)
    st = load_library().ulysses_attn_merge(
        _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), N, bs, heads, hd, _dtype_code(o_a),
        _ptr(o), _ptr(lse), _stream(stream))
    _check("ulysses_attn_merge", st)


def ulysses_attn_fwd_fused(q_chunks, k_chunks, v_chunks, o_chunks, lse, rank: int,
                           softmax_scale: float, causal: bool = True, cu_seqlens=None,
                           stream=None) -> None:
    """Forward with the exchange fused in: q_chunks, o_chunks are P tensors
    [n_local, bs, hq, hd] (all heads), k_chunks, v_chunks P tensors
    [n_local, bs, hkv, hd]; lse: fp32 [bs, hq/P, P*n_local].  Writes only this
    rank's head slots of o_chunks."""
    import torch
    P, n, bs, hq, hd = _need_chunks("q_chunks", q_chunks)
    hkv = _need_chunks("k_chunks", k_chunks, dtype=q_chunks[0].dtype)[3]
    for name, chunks, h in (("k_chunks", k_chunks, hkv), ("v_chunks", v_chunks, hkv),
                            ("o_chunks", o_chunks, hq)):
        if _need_chunks(name, chunks, h, q_chunks[0].dtype)[:3] != (P, n, bs) or \
                chunks[0].shape[3] != hd:
            raise ValueError(f"{name}: chunks differ from q_chunks in P, n_local, bs or head_dim")
    if hq % P == 0:   # otherwise the library reports ERR_DIVISIBILITY
        _need("lse", lse, (bs, hq // P, P * n), torch.float32)
    _need_cu(cu_seqlens)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    st = load_library().ulysses_attn_fwd_fused(
        _ptr_array(q_chunks), _ptr_array(k_chunks), _ptr_array(v_chunks), len(q_chunks), rank, n,
        bs, hq, hkv, hd, _dtype_code(q_chunks[0]), softmax_scale, int(causal), _ptr(cu_seqlens),
        n_docs, _ptr_array(o_chunks), _ptr(lse), _stream(stream))
    _check("ulysses_attn_fwd_fused", st)


def ulysses_attn_bwd_fused(q_chunks, k_chunks, v_chunks, o_chunks, lse, do_chunks, dq_chunks,
                           dk_chunks, dv_chunks, workspace, rank: int, softmax_scale: float,
                           causal: bool = True, cu_seqlens=None, stream=None) -> None:
    """Backward with the exchange fused in: every *_chunks argument is P
    tensors [n_local, bs, H, hd] (H = hq for q, o, do, dq; hkv for k, v, dk,
    dv); lse: fp32 [bs, hq/P, P*n_local] from ulysses_attn_fwd_fused;
    workspace as for ulysses_attn_bwd at the rank's head counts.  Writes only
    this rank's head slots of dq_chunks, dk_chunks and dv_chunks."""
    import torch
    P, n, bs, hq, hd = _need_chunks("q_chunks", q_chunks)
    hkv = _need_chunks("k_chunks", k_chunks, dtype=q_chunks[0].dtype)[3]
    for name, chunks, h in (("k_chunks", k_chunks, hkv), ("v_chunks", v_chunks, hkv),
                            ("o_chunks", o_chunks, hq), ("do_chunks", do_chunks, hq),
                            ("dq_chunks", dq_chunks, hq), ("dk_chunks", dk_chunks, hkv),
                            ("dv_chunks", dv_chunks, hkv)):
        if _need_chunks(name, chunks, h, q_chunks[0].dtype)[:3] != (P, n, bs) or \
                chunks[0].shape[3] != hd:
            raise ValueError(f"{name}: chunks differ from q_chunks in P, n_local, bs or head_dim")
    if hq % P == 0:
        _need("lse", lse, (bs, hq // P, P * n), torch.float32)
    _need_cu(cu_seqlens)
    _need_workspace(workspace)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().ulysses_attn_bwd_fused(
        _ptr_array(q_chunks), _ptr_array(k_chunks), _ptr_array(v_chunks), _ptr_array(o_chunks),
        _ptr(lse), _ptr_array(do_chunks), len(q_chunks), rank, n, bs, hq, hkv, hd,
        _dtype_code(q_chunks[0]), softmax_scale, int(causal), _ptr(cu_seqlens), n_docs,
        _ptr_array(dq_chunks), _ptr_array(dk_chunks), _ptr_array(dv_chunks), _ptr(workspace),
        ws_bytes, _stream(stream))
    _check("ulysses_attn_bwd_fused", st)


IGNORE_INDEX = -100


def ulysses_logits_loss_workspace_size(shard_rows: int, vocab: int) -> int:
    return int(load_library().ulysses_logits_loss_workspace_size(shard_rows, vocab))


def ulysses_logits_loss(h, w, labels, loss_rows, loss_sum, n_good, dh, dw, workspace,
                        grad_scale: float = 1.0, shard_rows: int = 4096,
                        ignore_index: int = IGNORE_INDEX, stream=None) -> None:
    """Language-model loss with the logits formed shard_rows rows at a time.
    h: bf16 [T, d]; w: bf16 [V, d]; labels: int64 [T]; loss_rows: fp32 [T];
    loss_sum: fp32 [1]; n_good: int64 [1]; dh: bf16 [T, d]; dw: fp32 [V, d];
    workspace: at least ulysses_logits_loss_workspace_size(min(shard_rows, T), V) bytes."""
    import torch
    if not isinstance(h, torch.Tensor) or h.dim() != 2 or not isinstance(w, torch.Tensor) or \
            w.dim() != 2:
        raise ValueError("h and w must be 2-D tensors [T, d] and [V, d]")
    T, d = h.shape
    V = w.shape[0]
    _need("h", h, (T, d))
    _need("w", w, (V, d), h.dtype)
    _need("labels", labels, (T,), torch.int64)
    _need("loss_rows", loss_rows, (T,), torch.float32)
    _need("loss_sum", loss_sum, (1,), torch.float32)
    _need("n_good", n_good, (1,), torch.int64)
    _need("dh", dh, (T, d), h.dtype)
    _need("dw", dw, (V, d), torch.float32)
    _need_workspace(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().ulysses_logits_loss(
        _ptr(h), _ptr(w), _ptr(labels), T, d, V, _dtype_code(h), ignore_index, grad_scale,
        shard_rows, _ptr(loss_rows), _ptr(loss_sum), _ptr(n_good), _ptr(dh), _ptr(dw),
        _ptr(workspace), ws_bytes, _stream(stream))
    _check("ulysses_logits_loss", st)


def ulysses_tiled_mlp_workspace_size(shard_rows: int, d: int, inter: int, backward: bool) -> int:
    return int(load_library().ulysses_tiled_mlp_workspace_size(shard_rows, d, inter, int(backward)))


def _need_mlp(x, wg, wu, wd):
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not isinstance(wg, torch.Tensor) or \
            wg.dim() != 2:
        raise ValueError("x and wg must be 2-D tensors [T, d] and [I, d]")
    T, d = x.shape
    inter = wg.shape[0]
    _need("x", x, (T, d))
    _need("wg", wg, (inter, d), x.dtype)
    _need("wu", wu, (inter, d), x.dtype)
    _need("wd", wd, (d, inter), x.dtype)
    return T, d, inter


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def ulysses_tiled_mlp_fwd(x, wg, wu, wd, y, workspace, shard_rows=None, stream=None) -> None:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T, shard_rows rows at a time (default
    d, the guide's ceil(T / d) shards).  x, y: bf16 [T, d]; wg, wu: [I, d];
    wd: [d, I]."""
    T, d, inter = _need_mlp(x, wg, wu, wd)
    _need("y", y, (T, d), x.dtype)
    _need_workspace(workspace)
    st = load_library().ulysses_tiled_mlp_fwd(
        _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), T, d, inter, _dtype_code(x),
        d if shard_rows is None else shard_rows, _ptr(y), _ptr(workspace), _nbytes(workspace),
        _stream(stream))
    _check("ulysses_tiled_mlp_fwd", st)


def ulysses_tiled_mlp_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, workspace, shard_rows=None,
                          stream=None) -> None:
    """Gradients of ulysses_tiled_mlp_fwd for dy (bf16 [T, d]): dx bf16 [T, d];
    dwg, dwu fp32 [I, d]; dwd fp32 [d, I]."""
    import torch
    T, d, inter = _need_mlp(x, wg, wu, wd)
    _need("dy", dy, (T, d), x.dtype)
    _need("dx", dx, (T, d), x.dtype)
    _need("dwg", dwg, (inter, d), torch.float32)
    _need("dwu", dwu, (inter, d), torch.float32)
    _need("dwd", dwd, (d, inter), torch.float32)
    _need_workspace(workspace)
    st = load_library().ulysses_tiled_mlp_bwd(
        _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(dy), T, d, inter, _dtype_code(x),
        d if shard_rows is None else shard_rows, _ptr(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd),
        _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("ulysses_tiled_mlp_bwd", st)
