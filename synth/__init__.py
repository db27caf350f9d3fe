"""Seeded synthetic inputs shared by the oracle and the GPU path.

Holds no attention or layout arithmetic: it maps (seed, stream, element index)
to numbers with a counter-based SplitMix64 generator and Box-Muller normals
(see ``synth.c`` for the exact definition), draws document lengths, and
describes the workloads (shapes, dtypes, seeds).

Element ``e`` of a generated tensor is counter ``offset + e`` of its stream,
with ``e`` the row-major flat index, so any slice can be produced on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
# The host-sanitizer test (tests/test_sanitizers.py) loads an instrumented
# build of synth.c through this; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("ULYSSES_SYNTH_LIB")
_lib = None

# Stream ids of the seeded inputs.
STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_DOCS = 1, 2, 3, 4, 5
# Streams of the language-model loss inputs: hidden states, lm_head weight,
# labels and the choice of ignored tokens.
STREAM_HIDDEN, STREAM_LM_HEAD, STREAM_LABELS, STREAM_IGNORE = 6, 7, 8, 9
# Streams of the MLP weights (gate_proj, up_proj, down_proj).
STREAM_MLP_GATE, STREAM_MLP_UP, STREAM_MLP_DOWN = 10, 11, 12
IGNORE_INDEX = -100


def lm_labels(seed: int, T: int, vocab: int, ignore_percent: int = 10) -> np.ndarray:
    """Seeded int64 labels in [0, vocab); about ignore_percent% of them are
    IGNORE_INDEX (token i is ignored when draw i of STREAM_IGNORE in
    [0, 100) falls below ignore_percent)."""
    labels = uniform_int(seed, STREAM_LABELS, T, 0, vocab - 1)
    drop = uniform_int(seed, STREAM_IGNORE, T, 0, 99) < ignore_percent
    labels[drop] = IGNORE_INDEX
    return labels


def build_lib() -> str:
    """Compile ``libsynth.so`` with gcc (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.synth_words.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_splitmix64_sequence.argtypes = [u64, i64, vp]
    for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
        getattr(lib, name).argtypes = [u64, u64, u64, i64, dbl, vp]
    lib.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, i64, vp]
    for name in ("synth_words", "synth_splitmix64_sequence", "synth_normal_f64",
                 "synth_normal_f32", "synth_normal_bf16", "synth_uniform_int"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def words(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _load().synth_words(seed, stream, offset, count, out.ctypes.data)
    return out


def splitmix64_sequence(state: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _load().synth_splitmix64_sequence(state, count, out.ctypes.data)
    return out


def normal(seed: int, stream: int, shape, dtype: str = "f64", scale: float = 1.0,
           offset: int = 0) -> np.ndarray:
    """Seeded N(0,1)*scale of the given shape.

    dtype "f64" -> float64, "f32" -> float32 (RNE), "bf16" -> uint16 bf16 bit
    patterns (RNE from the fp32 value).
    """
    shape = tuple(int(s) for s in shape)
    count = int(np.prod(shape)) if shape else 1
    lib = _load()
    if dtype == "f64":
        out = np.empty(shape, dtype=np.float64)
        lib.synth_normal_f64(seed, stream, offset, count, scale, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(seed, stream, offset, count, scale, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(seed, stream, offset, count, scale, out.ctypes.data)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def uniform_int(seed: int, stream: int, count: int, lo: int, hi: int, offset: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    _load().synth_uniform_int(seed, stream, offset, count, lo, hi, out.ctypes.data)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of generated storage (bf16 bits, f32 or f64)."""
    if dtype == "bf16":
        return bf16_to_f64(arr)
    return arr.astype(np.float64)


def doc_lengths(seed: int, total: int, lo: int = 512, hi: int = 16384) -> list:
    """Document lengths drawn uniformly in [lo, hi] until they sum to ``total``.

    Draw k is counter k of the documents stream; when a draw would reach or
    pass the remaining length, the last document takes the remainder (which
    may be shorter than ``lo``).
    """
    lengths = []
    pos = 0
    k = 0
    while pos < total:
        draw = int(uniform_int(seed, STREAM_DOCS, 1, lo, hi, offset=k)[0])
        k += 1
        if pos + draw >= total:
            draw = total - pos
        lengths.append(draw)
        pos += draw
    return lengths


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclass(frozen=True)
class Workload:
    """One rank's share of an Ulysses attention layer.

    ``hq``/``hkv`` are the global head counts held by every seq-sharded
    chunk; P ranks each own ``hq // P`` query heads after the exchange.
    ``q_prescale`` multiplies the generated Q values; ``softmax_scale`` is
    what the attention applies to q.k.
    """
    name: str
    seqlen: int          # full sequence N after the exchange
    P: int               # sequence-parallel degree (number of chunks)
    rank: int            # the rank whose share is computed
    bs: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str           # "bf16" or "f32"
    q_prescale: float
    softmax_scale: float
    seed: int
    docs: bool = False
    backward: bool = False
    head_sharded_inputs: bool = False   # inputs generated already head-sharded
    notes: str = field(default="", compare=False)

    @property
    def n_local(self) -> int:
        return self.seqlen // self.P

    @property
    def hq_local(self) -> int:
        return self.hq // self.P if self.hq >= self.P else 1

    @property
    def hkv_local(self) -> int:
        return self.hkv // self.P if self.hkv >= self.P else 1

    def doc_lengths(self):
        if not self.docs:
            return [self.seqlen]
        return doc_lengths(self.seed, self.seqlen)

    def cu_seqlens(self):
        return cu_seqlens_from_lengths(self.doc_lengths()) if self.docs else None

    def causal_pairs(self) -> int:
        """Allowed (i, j) pairs per query head under the causal (doc) mask."""
        return sum(L * (L + 1) // 2 for L in self.doc_lengths())

    def seq_tensor(self, stream: int, heads: int, scale: float = 1.0, rows=None) -> np.ndarray:
        """Seq-sharded global tensor [N, bs, heads, head_dim] (chunk c is rows
        [c*n, (c+1)*n)).  ``rows=(r0, r1)`` generates only that row range."""
        r0, r1 = (0, self.seqlen) if rows is None else rows
        per_row = self.bs * heads * self.head_dim
        return normal(self.seed, stream, (r1 - r0, self.bs, heads, self.head_dim),
                      dtype=self.dtype, scale=scale, offset=r0 * per_row)

    def head_tensor(self, stream: int, heads_local: int, scale: float = 1.0) -> np.ndarray:
        """Head-sharded tensor [N, bs, heads_local, head_dim] generated directly."""
        return normal(self.seed, stream, (self.seqlen, self.bs, heads_local, self.head_dim),
                      dtype=self.dtype, scale=scale)


WORKLOADS = {
    "tiny-p2": Workload(
        name="tiny-p2", seqlen=256, P=2, rank=0, bs=1, hq=4, hkv=4, head_dim=64,
        dtype="f32", q_prescale=1.0, softmax_scale=1.0 / 8.0, seed=1001, backward=True,
        notes="emulated P=2 rank, fp32, both ranks assembled"),
    "llama8b-share-32k": Workload(
        name="llama8b-share-32k", seqlen=32768, P=8, rank=3, bs=1, hq=32, hkv=8,
        head_dim=128, dtype="bf16", q_prescale=1.0 / np.sqrt(128.0), softmax_scale=1.0,
        seed=1002, notes="Llama-8B-shaped rank share at P=8"),
    "llama8b-share-128k": Workload(
        name="llama8b-share-128k", seqlen=131072, P=8, rank=3, bs=1, hq=32, hkv=8,
        head_dim=128, dtype="bf16", q_prescale=1.0 / np.sqrt(128.0), softmax_scale=1.0,
        seed=1003, backward=True, notes="8 chunks of 16384 tokens; fwd+bwd"),
    "long-256k": Workload(
        name="long-256k", seqlen=262144, P=1, rank=0, bs=1, hq=4, hkv=1, head_dim=128,
        dtype="bf16", q_prescale=1.0, softmax_scale=1.0 / np.sqrt(128.0), seed=1004,
        head_sharded_inputs=True, notes="fwd only, inputs already head-sharded"),
    "packed-docs-64k": Workload(
        name="packed-docs-64k", seqlen=65536, P=8, rank=3, bs=1, hq=32, hkv=8,
        head_dim=128, dtype="bf16", q_prescale=1.0, softmax_scale=1.0 / np.sqrt(128.0),
        seed=1005, docs=True, backward=True,
        notes="packed documents, lengths U{512..16384}, block-diagonal causal mask"),
}
