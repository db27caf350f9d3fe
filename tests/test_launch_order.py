"""The dispatch order of packed-document blocks (doc_sorted_block in
csrc/device_common.h), modelled on the host.

The device function computes, per workgroup, which block runs at launch rank
t: blocks sorted by a per-document key (query blocks: index from the block
holding the document's start; key blocks: distance to the document's last
block), largest first, documents in order within a key.  A rank found by a
binary search over the key and a pick among the documents must give every
block exactly once, or some outputs would never be written.  This model
follows the device function step for step (per-document ranges, the count
C(j) of blocks with key >= j, the search, the pick) and checks, for many
document sets, that the ranks form a permutation, that the order is by
non-increasing key, and when the device falls back to the positional order.
The GPU parity tests (every element of ragged, aligned, 256- and
301-document cases) check the device code itself.
"""
import random

import pytest

ORDER_DOCS = 256


def doc_ranges(cu, N, B, nblocks, key_blocks):
    """Owned blocks [f, l] and start block a per document, as on the device."""
    out = []
    for d in range(len(cu) - 1):
        s = min(max(cu[d], 0), N)
        e = min(max(cu[d + 1], s), N)
        if key_blocks:   # blocks whose last key lies in [s, e)
            f = s // B
            l = f - 1 if e <= s else (nblocks - 1 if e >= N else e // B - 1)
            a = 0
        else:            # blocks whose first position lies in [s, e)
            f = -(-s // B)
            l = -(-e // B) - 1
            a = s // B
        out.append((f, min(l, nblocks - 1), a))
    return out


def sorted_block(t, nblocks, B, cu, N, key_blocks):
    if len(cu) - 1 > ORDER_DOCS:
        return -1
    docs = doc_ranges(cu, N, B, nblocks, key_blocks)
    tops = [(l - f) if key_blocks else (l - a) for f, l, a in docs if l >= f]
    jmax = max(tops) if tops else -1

    def count_ge(j):
        c = 0
        for f, l, a in docs:
            lo = f if key_blocks else max(f, a + j)
            hi = l - j if key_blocks else l
            c += hi - lo + 1 if hi >= lo else 0
        return c

    if jmax < 0 or count_ge(0) <= t:
        return -1
    lo, hi = 0, jmax
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if count_ge(mid) > t:
            lo = mid
        else:
            hi = mid - 1
    r = t - count_ge(lo + 1)
    for f, l, a in docs:
        kb = l - lo if key_blocks else a + lo
        if l >= f and f <= kb <= l:
            if r == 0:
                return kb
            r -= 1
    return -1


def key_of(kb, cu, N, B, nblocks, key_blocks):
    for f, l, a in doc_ranges(cu, N, B, nblocks, key_blocks):
        if f <= kb <= l:
            return (l - kb) if key_blocks else (kb - a)
    raise AssertionError(kb)


def random_cu(rng, N, n_docs):
    cuts = sorted(rng.sample(range(1, N), n_docs - 1)) if n_docs > 1 else []
    return [0] + cuts + [N]


CASES = [
    (3005, [0, 1, 64, 128, 193, 320, 449, 578, 1278, 1279, 1280, 1282, 2282, 2582, 2589, 2597,
            2606, 3005]),
    (4096, [0, 512, 1536, 1792, 4096]),      # block-aligned
    (131072, [0, 131072]),                   # one document: the positional order
    (65536, [0, 3493, 13347, 23536, 37257, 51920, 62419, 64658, 65536]),
    (1, [0, 1]),
]


@pytest.mark.parametrize("B,key_blocks", [(64, False), (128, True)])
def test_order_is_a_heaviest_first_permutation(B, key_blocks):
    rng = random.Random(11)
    cases = list(CASES)
    for _ in range(200):
        N = rng.randint(1, 6000)
        cases.append((N, random_cu(rng, N, rng.randint(1, min(N, 40)))))
    for N, cu in cases:
        nb = -(-N // B)
        order = [sorted_block(t, nb, B, cu, N, key_blocks) for t in range(nb)]
        assert sorted(order) == list(range(nb)), (N, cu)
        keys = [key_of(kb, cu, N, B, nb, key_blocks) for kb in order]
        assert all(keys[i] >= keys[i + 1] for i in range(nb - 1)), (N, cu)


def test_one_document_keeps_the_positional_order():
    N, B = 131072, 64
    nb = N // B
    assert [sorted_block(t, nb, B, [0, N], N, False) for t in range(nb)] == list(range(nb))[::-1]
    nk = N // 128
    assert [sorted_block(t, nk, 128, [0, N], N, True) for t in range(nk)] == list(range(nk))


def test_falls_back_beyond_the_document_limit_or_on_bad_offsets():
    N = 2600
    cu = [7 * i for i in range(301)] + [N]                  # 301 documents
    assert sorted_block(0, -(-N // 64), 64, cu, N, False) == -1
    # offsets that cover no block: the device keeps its default order
    assert sorted_block(0, 4, 64, [0, 0], 256, False) == -1
