"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
the pages' two-GPU layout diagram, library routines that compute the same
definition by another route (numpy slicing, torch's fp64 scaled-dot-product
attention, torch autograd), closed forms, invariants and finite differences.
A plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one mask) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261202)


def rand(*shape):
    return RNG.standard_normal(shape)


def doc_ids(cu, N):
    return np.searchsorted(np.asarray(cu), np.arange(N), side="right") - 1


def allowed_mask(N, causal, cu):
    """Boolean [N, N] mask (query, key) built from positions and document ids."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    m = np.ones((N, N), dtype=bool)
    if causal:
        m &= j <= i
    if cu is not None:
        d = doc_ids(cu, N)
        m &= d[:, None] == d[None, :]
    return m


def sdpa_reference(q, k, v, scale, causal, cu):
    """torch's fp64 scaled_dot_product_attention; layout [N, bs, H, hd]."""
    tq = torch.from_numpy(q).permute(1, 2, 0, 3)
    tk = torch.from_numpy(k).permute(1, 2, 0, 3)
    tv = torch.from_numpy(v).permute(1, 2, 0, 3)
    mask = torch.from_numpy(allowed_mask(q.shape[0], causal, cu))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=q.shape[2] != k.shape[2])
    return out.permute(2, 0, 1, 3).numpy()


def explicit_attention_torch(q, k, v, scale, causal, cu):
    """Scores -> masked softmax -> weighted values, by torch tensor ops (fp64);
    returns (O, LSE, autograd-ready leaf tensors)."""
    N, bs, hq, hd = q.shape
    g = hq // k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kr = tk.repeat_interleave(g, dim=2)
    vr = tv.repeat_interleave(g, dim=2)
    s = torch.einsum("ibhe,jbhe->bhij", tq, kr) * scale
    mask = torch.from_numpy(allowed_mask(N, causal, cu))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                       # [bs, hq, N]
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,jbhe->ibhe", p, vr)
    return o, lse, (tq, tk, tv)


# --------------------------------------------------------------------------
# Layout exchange
# --------------------------------------------------------------------------

def test_layout_matches_two_gpu_diagram():
    fx = json.load(open(os.path.join(GOLDEN, "layout_2gpu_diagram.json")))
    chunks = [np.asarray(fx["seq_sharded"][f"gpu{c}"], dtype=np.int32)[:, None, :, None]
              for c in range(fx["P"])]
    for r in range(fx["P"]):
        got = oracle.seq_to_head(chunks, r)
        want = np.asarray(fx["head_sharded"][f"gpu{r}"], dtype=np.int32)[:, None, :, None]
        np.testing.assert_array_equal(got, want)
    back = [np.full_like(c, -1) for c in chunks]
    for r in range(fx["P"]):
        x = np.asarray(fx["head_sharded"][f"gpu{r}"], dtype=np.int32)[:, None, :, None].copy()
        oracle.head_to_seq(x, back, r)
    for c in range(fx["P"]):
        np.testing.assert_array_equal(back[c], chunks[c])


@pytest.mark.parametrize("P,heads,bs,n,hd,dtype", [
    (2, 4, 1, 8, 16, np.float32), (4, 8, 2, 5, 8, np.uint16), (8, 32, 1, 3, 4, np.uint16),
    (8, 8, 1, 4, 128, np.uint16), (1, 3, 2, 6, 4, np.float64)])
def test_seq_to_head_is_concat_then_head_slice(P, heads, bs, n, hd, dtype):
    hl = heads // P
    chunks = [RNG.integers(0, 60000, size=(n, bs, heads, hd)).astype(dtype) for _ in range(P)]
    full = np.concatenate(chunks, axis=0)
    for r in range(P):
        got = oracle.seq_to_head(chunks, r)
        np.testing.assert_array_equal(got, full[:, :, r * hl:(r + 1) * hl, :])
        assert got.tobytes() == np.ascontiguousarray(full[:, :, r * hl:(r + 1) * hl, :]).tobytes()


@pytest.mark.parametrize("P,heads", [(8, 2), (4, 1), (8, 4), (2, 1)])
def test_seq_to_head_replicates_kv_when_heads_below_P(P, heads):
    chunks = [RNG.integers(0, 1000, size=(3, 1, heads, 4)).astype(np.int16) for _ in range(P)]
    full = np.concatenate(chunks, axis=0)
    for r in range(P):
        got = oracle.seq_to_head(chunks, r)
        src = (r * heads) // P
        np.testing.assert_array_equal(got, full[:, :, src:src + 1, :])


@pytest.mark.parametrize("P,heads", [(8, 12), (3, 4), (8, 3)])
def test_seq_to_head_rejects_indivisible_heads(P, heads):
    chunks = [np.zeros((2, 1, heads, 4), np.float32) for _ in range(P)]
    with pytest.raises(ValueError):
        oracle.seq_to_head(chunks, 0)


@pytest.mark.parametrize("P,heads,bs", [(2, 4, 1), (4, 8, 2), (8, 32, 1)])
def test_round_trip_over_all_ranks_is_identity_and_touches_only_own_slots(P, heads, bs):
    n, hd = 5, 8
    hl = heads // P
    chunks = [RNG.integers(0, 65535, size=(n, bs, heads, hd)).astype(np.uint16) for _ in range(P)]
    canary = np.uint16(0xDEAD)
    back = [np.full_like(c, canary) for c in chunks]
    for r in range(P):
        oracle.head_to_seq(oracle.seq_to_head(chunks, r), back, r)
        for c in range(P):
            owned = back[c][:, :, : (r + 1) * hl, :]
            np.testing.assert_array_equal(owned, chunks[c][:, :, : (r + 1) * hl, :])
            assert np.all(back[c][:, :, (r + 1) * hl:, :] == canary)
    for c in range(P):
        assert back[c].tobytes() == chunks[c].tobytes()


def test_single_rank_exchange_is_identity():
    x = RNG.integers(0, 65535, size=(7, 2, 3, 4)).astype(np.uint16)
    np.testing.assert_array_equal(oracle.seq_to_head([x], 0), x)


# --------------------------------------------------------------------------
# Attention forward
# --------------------------------------------------------------------------

FWD_CASES = [
    # N, bs, hq, hkv, hd, scale, causal, cu
    (1, 1, 2, 2, 8, 0.35, True, None),
    (7, 1, 2, 2, 8, 0.35, True, None),
    (33, 2, 4, 1, 16, 0.25, True, None),
    (40, 1, 4, 2, 8, 1.0, True, None),
    (64, 1, 2, 1, 16, 0.125, True, [0, 1, 20, 21, 64]),
    (30, 2, 2, 2, 8, 0.5, False, None),
    (30, 1, 4, 2, 8, 0.5, False, [0, 11, 12, 30]),
]


@pytest.mark.parametrize("N,bs,hq,hkv,hd,scale,causal,cu", FWD_CASES)
def test_fwd_matches_torch_sdpa_and_logsumexp(N, bs, hq, hkv, hd, scale, causal, cu):
    q, k, v = rand(N, bs, hq, hd), rand(N, bs, hkv, hd), rand(N, bs, hkv, hd)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, cu)
    np.testing.assert_allclose(o, sdpa_reference(q, k, v, scale, causal, cu), rtol=1e-11, atol=1e-12)
    _, lse_t, _ = explicit_attention_torch(q, k, v, scale, causal, cu)
    np.testing.assert_allclose(lse, lse_t.detach().numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cu", [None, [0, 5, 6, 17, 40]])
def test_fwd_zero_q_gives_prefix_mean_and_log_count(cu):
    N, hd = 40, 8
    q = np.zeros((N, 1, 2, hd))
    k, v = rand(N, 1, 1, hd), rand(N, 1, 1, hd)
    o, lse = oracle.attn_fwd(q, k, v, 0.7, True, cu)
    starts = np.zeros(N, dtype=int) if cu is None else np.asarray(cu)[doc_ids(cu, N)]
    for i in range(N):
        mean = v[starts[i]:i + 1, 0, 0, :].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(o[i, 0, h], mean, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, h, i] - np.log(i - starts[i] + 1)) < 1e-12


def test_fwd_constant_v_returns_v():
    N, hd = 50, 16
    q, k = rand(N, 2, 4, hd), rand(N, 2, 2, hd)
    row = rand(hd)
    v = np.broadcast_to(row, (N, 2, 2, hd)).copy()
    o, _ = oracle.attn_fwd(q, k, v, 0.3, True, [0, 13, 50])
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-12, atol=1e-12)


def test_fwd_single_token_returns_its_value_and_score():
    q, k, v = rand(1, 1, 3, 8), rand(1, 1, 3, 8), rand(1, 1, 3, 8)
    o, lse = oracle.attn_fwd(q, k, v, 0.9, True)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], 0.9 * np.sum(q[0, 0] * k[0, 0], axis=-1), rtol=1e-14)


def test_fwd_gqa_equals_mha_with_repeated_kv():
    N, hd, g = 37, 8, 4
    q, k, v = rand(N, 1, 8, hd), rand(N, 1, 2, hd), rand(N, 1, 2, hd)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.4, True)
    o2, l2 = oracle.attn_fwd(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), 0.4, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_fwd_documents_are_independent_attentions():
    cu = [0, 9, 10, 31, 48]
    N, hd = 48, 8
    q, k, v = rand(N, 1, 2, hd), rand(N, 1, 1, hd), rand(N, 1, 1, hd)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        od, ld = oracle.attn_fwd(q[a:b], k[a:b], v[a:b], 0.5, True)
        np.testing.assert_allclose(o[a:b], od, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, a:b], ld, rtol=1e-13, atol=1e-14)


def test_fwd_sampled_rows_equal_full_rows():
    N, hd = 45, 8
    cu = [0, 20, 45]
    q, k, v = rand(N, 2, 2, hd), rand(N, 2, 1, hd), rand(N, 2, 1, hd)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True, cu)
    rows = [44, 0, 19, 20, 7]
    os_, ls = oracle.attn_fwd(q, k, v, 0.5, True, cu, rows=rows)
    np.testing.assert_array_equal(os_, o[rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])


@pytest.mark.parametrize("P,hq,hkv", [(2, 4, 4), (4, 8, 4), (4, 8, 2)])
def test_head_sharded_share_equals_full_mha_restricted_to_rank_heads(P, hq, hkv):
    """Heads are independent, so running every rank's share (exchange,
    local attention on hq/P heads, inverse exchange) rebuilds full
    multi-head attention."""
    N, hd, n = 24, 8, 24 // P
    q, k, v = rand(N, 1, hq, hd), rand(N, 1, hkv, hd), rand(N, 1, hkv, hd)
    o_full, _ = oracle.attn_fwd(q, k, v, 0.6, True)
    qc = [np.ascontiguousarray(q[c * n:(c + 1) * n]) for c in range(P)]
    kc = [np.ascontiguousarray(k[c * n:(c + 1) * n]) for c in range(P)]
    vc = [np.ascontiguousarray(v[c * n:(c + 1) * n]) for c in range(P)]
    oc = [np.full((n, 1, hq, hd), np.nan) for _ in range(P)]
    for r in range(P):
        ql, kl, vl = oracle.seq_to_head(qc, r), oracle.seq_to_head(kc, r), oracle.seq_to_head(vc, r)
        ol, _ = oracle.attn_fwd(ql, kl, vl, 0.6, True)
        oracle.head_to_seq(np.ascontiguousarray(ol), oc, r)
    np.testing.assert_allclose(np.concatenate(oc, axis=0), o_full, rtol=1e-13, atol=1e-14)


def test_fwd_rejects_bad_documents():
    q = rand(8, 1, 1, 4)
    for cu in ([0, 4, 7], [1, 8], [0, 4, 4, 8]):
        with pytest.raises(ValueError):
            oracle.attn_fwd(q, q, q, 1.0, True, cu)


# --------------------------------------------------------------------------
# Attention backward
# --------------------------------------------------------------------------

BWD_CASES = [
    (9, 1, 2, 2, 8, 0.4, True, None),
    (33, 2, 4, 1, 8, 0.25, True, None),
    (40, 1, 4, 2, 16, 1.3, True, [0, 1, 17, 18, 40]),
    (21, 1, 2, 1, 8, 0.5, False, [0, 8, 21]),
]


@pytest.mark.parametrize("N,bs,hq,hkv,hd,scale,causal,cu", BWD_CASES)
def test_bwd_matches_torch_autograd(N, bs, hq, hkv, hd, scale, causal, cu):
    q, k, v = rand(N, bs, hq, hd), rand(N, bs, hkv, hd), rand(N, bs, hkv, hd)
    do = rand(N, bs, hq, hd)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal, cu)
    o, _, (tq, tk, tv) = explicit_attention_torch(q, k, v, scale, causal, cu)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_bwd_matches_central_finite_differences():
    N, hd = 12, 4
    cu = [0, 5, 12]
    q, k, v = rand(N, 1, 2, hd), rand(N, 1, 1, hd), rand(N, 1, 1, hd)
    do = rand(N, 1, 2, hd)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.8, True, cu)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, 0.8, True, cu)
        return float(np.sum(o * do))

    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0, 1), (4, 0, 0, 3), (5, 0, 0, 0), (11, 0, x.shape[2] - 1, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-8 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_bwd_constant_v_has_zero_dq_dk_and_constant_k_has_zero_dq():
    N, hd = 30, 8
    q, k = rand(N, 1, 2, hd), rand(N, 1, 1, hd)
    row = rand(hd)
    vconst = np.broadcast_to(row, (N, 1, 1, hd)).copy()
    do = rand(N, 1, 2, hd)
    dq, dk, _ = oracle.attn_bwd(q, k, vconst, do, 0.5, True, [0, 10, 30])
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    kconst = np.broadcast_to(rand(hd), (N, 1, 1, hd)).copy()
    dq, _, _ = oracle.attn_bwd(q, kconst, rand(N, 1, 1, hd), do, 0.5, True)
    assert np.max(np.abs(dq)) < 1e-12


def test_bwd_column_sums_per_document():
    """Softmax is shift-invariant: sum_j dK_j = 0 in each document; and
    sum_j dV_j equals the group's summed dO over the document."""
    N, hd, cu = 36, 8, [0, 7, 8, 36]
    q, k, v = rand(N, 1, 4, hd), rand(N, 1, 2, hd), rand(N, 1, 2, hd)
    do = rand(N, 1, 4, hd)
    _, dk, dv = oracle.attn_bwd(q, k, v, do, 0.7, True, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        np.testing.assert_allclose(dk[a:b].sum(axis=0), 0.0, atol=1e-12)
        for kh in range(2):
            want = do[a:b, :, 2 * kh:2 * kh + 2].sum(axis=(0, 2))
            np.testing.assert_allclose(dv[a:b, :, kh].sum(axis=0), want, rtol=1e-12, atol=1e-12)


def test_bwd_zero_q_dv_closed_form():
    N, hd, cu = 25, 4, [0, 10, 25]
    q = np.zeros((N, 1, 2, hd))
    k, v, do = rand(N, 1, 1, hd), rand(N, 1, 1, hd), rand(N, 1, 2, hd)
    _, _, dv = oracle.attn_bwd(q, k, v, do, 1.0, True, cu)
    starts = np.asarray(cu)[doc_ids(cu, N)]
    ends = np.asarray(cu)[doc_ids(cu, N) + 1]
    for j in range(N):
        want = sum(do[i, 0, h] / (i - starts[i] + 1) for h in range(2) for i in range(j, ends[j]))
        np.testing.assert_allclose(dv[j, 0, 0], want, rtol=1e-12, atol=1e-12)


def test_bwd_sampled_rows_and_columns_equal_full():
    N, hd, cu = 30, 8, [0, 12, 30]
    q, k, v, do = rand(N, 2, 2, hd), rand(N, 2, 1, hd), rand(N, 2, 1, hd), rand(N, 2, 2, hd)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.5, True, cu)
    rows, cols = [29, 3, 12], [0, 11, 12, 29]
    sq, sk, sv = oracle.attn_bwd(q, k, v, do, 0.5, True, cu, dq_rows=rows, dkv_cols=cols)
    np.testing.assert_array_equal(sq, dq[rows])
    np.testing.assert_array_equal(sk, dk[cols])
    np.testing.assert_array_equal(sv, dv[cols])
    eq, ek, ev = oracle.attn_bwd(q, k, v, do, 0.5, True, cu, dq_rows=[], dkv_cols=cols)
    assert eq.shape[0] == 0
    np.testing.assert_array_equal(ek, dk[cols])


# --------------------------------------------------------------------------
# Inputs shared by both sides
# --------------------------------------------------------------------------

def test_splitmix64_matches_published_outputs():
    fx = json.load(open(os.path.join(GOLDEN, "splitmix64_1234567.json")))
    got = synth.splitmix64_sequence(fx["state"], len(fx["outputs"]))
    assert [int(x) for x in got] == [int(s) for s in fx["outputs"]]


def test_generated_normals_have_unit_moments_and_are_sliceable():
    x = synth.normal(7, 1, (400000,))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    part = synth.normal(7, 1, (1000,), offset=1234)
    np.testing.assert_array_equal(part, x[1234:2234])
    b = synth.normal(7, 1, (1000,), dtype="bf16", offset=1234)
    f = synth.normal(7, 1, (1000,), dtype="f32", offset=1234)
    np.testing.assert_array_equal(synth.bf16_to_f64(b), torch.from_numpy(f).to(torch.bfloat16).double().numpy())


def test_document_lengths_follow_the_recipe():
    for seed in (1005, 1, 2):
        lengths = synth.doc_lengths(seed, 65536)
        assert sum(lengths) == 65536
        assert all(512 <= L <= 16384 for L in lengths[:-1])
        assert 1 <= lengths[-1] <= 16384


# --------------------------------------------------------------------------
# Magnitudes (sum of |terms|) used to size rounding-error tolerances
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,cu", [(True, None), (True, [0, 9, 10, 30]), (False, [0, 12, 30])])
def test_magnitudes_match_torch_absolute_sums(causal, cu):
    """M = the output sum with every term replaced by its absolute value;
    dS_ij comes from torch autograd on the scores, P from torch.softmax."""
    N, hd, hq, hkv, scale = 30, 8, 4, 2, 0.6
    g = hq // hkv
    q, k, v, do = rand(N, 1, hq, hd), rand(N, 1, hkv, hd), rand(N, 1, hkv, hd), rand(N, 1, hq, hd)
    _, _, mo = oracle.attn_fwd(q, k, v, scale, causal, cu, magnitude=True)
    _, _, _, m = oracle.attn_bwd(q, k, v, do, scale, causal, cu, magnitude=True)
    mdq, mdk, mdv = m["dq"], m["dk"], m["dv"]
    mask = torch.from_numpy(allowed_mask(N, causal, cu))
    kr = torch.from_numpy(np.repeat(k[:, 0], g, axis=1))   # [N, hq, hd]
    vr = torch.from_numpy(np.repeat(v[:, 0], g, axis=1))
    tq, tdo = torch.from_numpy(q[:, 0]), torch.from_numpy(do[:, 0])
    s = (torch.einsum("ihe,jhe->hij", tq, kr) * scale).detach().requires_grad_(True)
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
    o = torch.einsum("hij,jhe->ihe", p, vr)
    o.backward(tdo)
    ds = s.grad.abs()                                        # [hq, N, N]
    pa = p.detach()
    want_mo = torch.einsum("hij,jhe->ihe", pa, vr.abs())
    want_mdq = scale * torch.einsum("hij,jhe->ihe", ds, kr.abs())
    want_mdk = scale * torch.einsum("hij,ihe->jhe", ds, tq.abs()).reshape(N, hkv, g, hd).sum(2)
    want_mdv = torch.einsum("hij,ihe->jhe", pa, tdo.abs()).reshape(N, hkv, g, hd).sum(2)
    np.testing.assert_allclose(mo[:, 0], want_mo.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(mdq[:, 0], want_mdq.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(mdk[:, 0], want_mdk.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(mdv[:, 0], want_mdv.numpy(), rtol=1e-11, atol=1e-12)
    # sensitivity to D: A_i = sum_e |dO_ie| (P |V|)_ie
    A = (tdo.abs() * want_mo).sum(-1)                        # [N, hq]
    want_dq_d = scale * A[:, :, None] * torch.einsum("hij,jhe->ihe", pa, kr.abs())
    want_dk_d = scale * torch.einsum("hij,ih,ihe->jhe", pa, A, tq.abs()).reshape(N, hkv, g, hd).sum(2)
    np.testing.assert_allclose(m["dq_from_D"][:, 0], want_dq_d.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(m["dk_from_D"][:, 0], want_dk_d.numpy(), rtol=1e-10, atol=1e-11)


def test_magnitudes_bound_the_values_and_equal_them_for_same_sign_terms():
    N, hd = 25, 8
    q, k = rand(N, 1, 2, hd), rand(N, 1, 1, hd)
    v_pos, do_pos = np.abs(rand(N, 1, 1, hd)), np.abs(rand(N, 1, 2, hd))
    o, _, mo = oracle.attn_fwd(q, k, v_pos, 0.5, True, magnitude=True)
    np.testing.assert_allclose(mo, o, rtol=1e-13)            # all terms positive
    dq, dk, dv, m = oracle.attn_bwd(q, k, v_pos, do_pos, 0.5, True, magnitude=True)
    mdq, mdk, mdv = m["dq"], m["dk"], m["dv"]
    np.testing.assert_allclose(mdv, dv, rtol=1e-13)
    assert np.all(mdq >= np.abs(dq) - 1e-12) and np.all(mdk >= np.abs(dk) - 1e-12)


def test_bwd_with_given_forward_outputs():
    """The backward as a call receives it: O and LSE passed in.  Passing the
    oracle's own values changes nothing; shifting O changes D_i by <dO_i, dO_>
    and moves dQ_i by -scale dD_i sum_j P_ij k_j (attention of q over k with
    values k) and dK_j by -scale sum_i P_ij dD_i q_i, leaving dV unchanged."""
    N, hd, cu, scale = 28, 8, [0, 11, 28], 0.7
    q, k, v, do = rand(N, 1, 2, hd), rand(N, 1, 1, hd), rand(N, 1, 1, hd), rand(N, 1, 2, hd)
    o, lse = oracle.attn_fwd(q, k, v, scale, True, cu)
    base = oracle.attn_bwd(q, k, v, do, scale, True, cu)
    same = oracle.attn_bwd(q, k, v, do, scale, True, cu, o=o, lse=lse)
    for a, b in zip(base, same):
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)
    delta = 0.01 * rand(N, 1, 2, hd)
    dq2, dk2, dv2 = oracle.attn_bwd(q, k, v, do, scale, True, cu, o=o + delta, lse=lse)
    dD = np.sum(do * delta, axis=-1)                         # [N, 1, 2]
    pk, _ = oracle.attn_fwd(q, k, k, scale, True, cu)        # sum_j P_ij k_j
    np.testing.assert_allclose(dq2 - base[0], -scale * dD[..., None] * pk, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dv2, base[2], rtol=1e-12, atol=1e-13)
    mask = allowed_mask(N, True, cu)
    want_dk = np.zeros_like(k)
    for h in range(2):
        s_ = scale * q[:, 0, h] @ k[:, 0, 0].T
        P = np.where(mask, np.exp(s_ - lse[0, h][:, None]), 0.0)
        want_dk[:, 0, 0] += -scale * P.T @ (dD[:, 0, h][:, None] * q[:, 0, h])
    np.testing.assert_allclose(dk2 - base[1], want_dk, rtol=1e-9, atol=1e-12)


# --- merge of partial results over disjoint key sets (ring / blockwise) ---

@pytest.mark.parametrize("hkv", [1, 2])
def test_merge_of_disjoint_key_blocks_equals_attention_over_their_union(hkv):
    n, bs, hq, hd, scale = 13, 2, 2, 8, 0.4
    q = rand(n, bs, hq, hd)
    ka, va, kb, vb = (rand(n, bs, hkv, hd) for _ in range(4))
    oa, la = oracle.attn_fwd(q, ka, va, scale, causal=False)
    ob, lb = oracle.attn_fwd(q, kb, vb, scale, causal=False)
    o, lse = oracle.attn_merge(oa, la, ob, lb)
    # the same queries against all 2n keys: stack the queries twice and read rows [0, n)
    full_o, full_l = oracle.attn_fwd(np.concatenate([q, q]), np.concatenate([ka, kb]),
                                     np.concatenate([va, vb]), scale, causal=False)
    np.testing.assert_allclose(o, full_o[:n], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, full_l[:, :, :n], rtol=1e-12, atol=1e-12)


def test_ring_steps_rebuild_causal_attention_of_the_second_block():
    # Rows [n, 2n) of causal attention over 2n positions: the first key block
    # is entirely visible (non-causal), the second is the causal diagonal.
    n, bs, hq, hkv, hd, scale = 11, 1, 4, 1, 16, 0.3
    q, k, v = rand(2 * n, bs, hq, hd), rand(2 * n, bs, hkv, hd), rand(2 * n, bs, hkv, hd)
    o1, l1 = oracle.attn_fwd(q[n:], k[:n], v[:n], scale, causal=False)
    o2, l2 = oracle.attn_fwd(q[n:], k[n:], v[n:], scale, causal=True)
    o, lse = oracle.attn_merge(o1, l1, o2, l2)
    full_o, full_l = oracle.attn_fwd(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o, full_o[n:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, full_l[:, :, n:], rtol=1e-12, atol=1e-12)


def test_merge_lse_is_numpy_logaddexp_and_weights_sum_to_one():
    N, bs, heads, hd = 7, 1, 3, 4
    la, lb = rand(bs, heads, N) * 30, rand(bs, heads, N) * 30
    oa, ob = rand(N, bs, heads, hd), rand(N, bs, heads, hd)
    o, lse = oracle.attn_merge(oa, la, ob, lb)
    np.testing.assert_allclose(lse, np.logaddexp(la, lb), rtol=1e-14, atol=1e-12)
    # merging O = 1 with O = 1 must give 1 whatever the statistics
    ones = np.ones_like(oa)
    o1, _ = oracle.attn_merge(ones, la, ones, lb)
    np.testing.assert_allclose(o1, 1.0, rtol=1e-14)
    # a partial with a far smaller LSE leaves the other almost unchanged
    o2, _ = oracle.attn_merge(oa, np.full_like(la, 10.0), ob, np.full_like(lb, -60.0))
    np.testing.assert_allclose(o2, oa, rtol=1e-12, atol=1e-25)


def test_merge_with_an_empty_partial_returns_the_other_and_empty_pair_is_zero():
    N, bs, heads, hd = 5, 2, 2, 3
    oa, la = rand(N, bs, heads, hd), rand(bs, heads, N)
    garbage = np.full((N, bs, heads, hd), np.nan)
    ninf = np.full((bs, heads, N), -np.inf)
    o, lse = oracle.attn_merge(oa, la, garbage, ninf)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)
    o, lse = oracle.attn_merge(garbage, ninf, oa, la)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)
    o, lse = oracle.attn_merge(garbage, ninf, garbage, ninf)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_merge_of_a_result_with_itself_keeps_o_and_adds_ln2():
    N, bs, heads, hd = 6, 1, 2, 5
    oa, la = rand(N, bs, heads, hd), rand(bs, heads, N)
    o, lse = oracle.attn_merge(oa, la, oa, la)
    np.testing.assert_allclose(o, oa, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(lse, la + np.log(2.0), rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------------------
# Language-model loss (lm_head + cross-entropy with ignored labels) and its
# gradients: the computation the integration guide's tiled fused logits loss
# shards over the sequence.
# ---------------------------------------------------------------------------

def lm_inputs(T, d, V, seed, ignore_every=4):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d)) / np.sqrt(d)
    labels = rng.integers(0, V, size=T)
    labels[::ignore_every] = oracle.IGNORE_INDEX
    return h, w, labels


@pytest.mark.parametrize("T,d,V,s", [(7, 5, 11, 1.0), (16, 8, 33, 0.25), (3, 16, 2, 1.0 / 3)])
def test_logits_loss_matches_torch_cross_entropy_and_autograd(T, d, V, s):
    """torch's own cross-entropy (sum over kept tokens, ignore_index) and its
    autograd gradients, in fp64 on the CPU."""
    h, w, labels = lm_inputs(T, d, V, seed=T * 100 + V)
    loss_rows, loss_sum, n_good, dh, dw = oracle.logits_loss(h, w, labels, s)
    ht = torch.tensor(h, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    lt = torch.tensor(labels)
    rows = torch.nn.functional.cross_entropy(ht @ wt.T, lt, ignore_index=oracle.IGNORE_INDEX,
                                             reduction="none")
    (s * rows.sum()).backward()
    np.testing.assert_allclose(loss_rows, rows.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert loss_sum == pytest.approx(float(rows.sum()), rel=1e-12, abs=1e-12)
    assert n_good == int((labels != oracle.IGNORE_INDEX).sum())
    np.testing.assert_allclose(dh, ht.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_logits_loss_zero_weights_closed_form():
    """W = 0: every logit is 0, so a kept token's loss is ln V, dh = 0, and
    dW_v = s * sum_i (1/V - [y_i = v]) h_i over kept tokens."""
    T, d, V, s = 9, 4, 6, 0.5
    h, _, labels = lm_inputs(T, d, V, seed=5)
    w = np.zeros((V, d))
    loss_rows, loss_sum, n_good, dh, dw = oracle.logits_loss(h, w, labels, s)
    kept = labels != oracle.IGNORE_INDEX
    np.testing.assert_allclose(loss_rows[kept], np.log(V), rtol=1e-14)
    assert np.all(loss_rows[~kept] == 0.0)
    assert loss_sum == pytest.approx(kept.sum() * np.log(V), rel=1e-14)
    assert np.all(dh == 0.0)
    expect = np.zeros((V, d))
    for i in np.nonzero(kept)[0]:
        expect += h[i] / V
        expect[labels[i]] -= h[i]
    np.testing.assert_allclose(dw, s * expect, rtol=1e-12, atol=1e-14)


def test_logits_loss_two_classes_is_logistic_loss():
    """V = 2: the loss is log(1 + e^(z_other - z_label)) (binary logistic)."""
    T, d = 12, 6
    h, w, _ = lm_inputs(T, d, 2, seed=8)
    labels = np.arange(T) % 2                       # every token kept
    loss_rows, *_ = oracle.logits_loss(h, w, labels)
    z = h @ w.T
    margin = z[np.arange(T), 1 - labels] - z[np.arange(T), labels]
    np.testing.assert_allclose(loss_rows, np.log1p(np.exp(margin)), rtol=1e-12)


def test_logits_loss_gradients_match_finite_differences():
    T, d, V, s = 4, 3, 5, 0.7
    h, w, labels = lm_inputs(T, d, V, seed=11)
    _, _, _, dh, dw = oracle.logits_loss(h, w, labels, s)
    eps = 1e-6

    def loss(hh, ww):
        return s * oracle.logits_loss(hh, ww, labels)[1]

    for (i, k) in [(0, 0), (1, 2), (3, 1)]:
        hp, hm = h.copy(), h.copy()
        hp[i, k] += eps
        hm[i, k] -= eps
        assert dh[i, k] == pytest.approx((loss(hp, w) - loss(hm, w)) / (2 * eps), abs=1e-7)
    for (v, k) in [(0, 0), (2, 1), (4, 2)]:
        wp, wm = w.copy(), w.copy()
        wp[v, k] += eps
        wm[v, k] -= eps
        assert dw[v, k] == pytest.approx((loss(h, wp) - loss(h, wm)) / (2 * eps), abs=1e-7)


def test_logits_loss_invariants():
    """Shifting every w_v by one vector shifts a row's logits equally: the
    losses stay.  The rows of G sum to zero, so sum_v dW_v = 0."""
    T, d, V = 10, 7, 13
    h, w, labels = lm_inputs(T, d, V, seed=21)
    rows, _, _, _, dw = oracle.logits_loss(h, w, labels)
    shifted, *_ = oracle.logits_loss(h, w + np.random.default_rng(2).standard_normal(d), labels)
    np.testing.assert_allclose(shifted, rows, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw.sum(axis=0), 0.0, atol=1e-12)


def test_logits_loss_all_ignored_and_bad_labels():
    h, w, _ = lm_inputs(4, 3, 5, seed=1)
    labels = np.full(4, oracle.IGNORE_INDEX)
    rows, total, n_good, dh, dw = oracle.logits_loss(h, w, labels)
    assert total == 0.0 and n_good == 0
    assert not rows.any() and not dh.any() and not dw.any()
    with pytest.raises(ValueError):
        oracle.logits_loss(h, w, np.array([0, 1, 5, 2]))        # label == V
    with pytest.raises(ValueError):
        oracle.logits_loss(h, w, np.array([0, -1, 2, 2]))       # negative, not the ignore index


# ---------------------------------------------------------------------------
# Sequence-tiled SwiGLU MLP (TiledMLP): y = (silu(x Wg^T) * (x Wu^T)) Wd^T.
# ---------------------------------------------------------------------------

def mlp_inputs(T, d, I, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.standard_normal((I, d)) / np.sqrt(d),
            rng.standard_normal((I, d)) / np.sqrt(d), rng.standard_normal((d, I)) / np.sqrt(I),
            rng.standard_normal((T, d)))


@pytest.mark.parametrize("T,d,I", [(5, 4, 7), (12, 8, 20), (1, 16, 3)])
def test_swiglu_mlp_matches_torch_autograd(T, d, I):
    x, wg, wu, wd, dy = mlp_inputs(T, d, I, seed=T + d + I)
    y, dx, dwg, dwu, dwd = oracle.swiglu_mlp(x, wg, wu, wd, dy)
    t = [torch.tensor(a, requires_grad=True) for a in (x, wg, wu, wd)]
    yt = (torch.nn.functional.silu(t[0] @ t[1].T) * (t[0] @ t[2].T)) @ t[3].T
    yt.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-13)
    for mine, ref in zip((dx, dwg, dwu, dwd), t):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_swiglu_mlp_zero_gate_closed_form():
    """Wg = 0: g = 0, silu(0) = 0 and silu'(0) = 1/2, so y = 0, dx = 0,
    dWu = 0, dWd = 0 and dWg = (1/2 (dy Wd) * u)^T x with u = x Wu^T."""
    x, _, wu, wd, dy = mlp_inputs(6, 5, 4, seed=3)
    wg = np.zeros_like(wu)
    y, dx, dwg, dwu, dwd = oracle.swiglu_mlp(x, wg, wu, wd, dy)
    assert not y.any() and not dx.any() and not dwu.any() and not dwd.any()
    u = x @ wu.T
    np.testing.assert_allclose(dwg, (0.5 * (dy @ wd) * u).T @ x, rtol=1e-12, atol=1e-14)


def test_swiglu_mlp_gradients_match_finite_differences():
    x, wg, wu, wd, dy = mlp_inputs(3, 4, 5, seed=9)
    _, dx, dwg, dwu, dwd = oracle.swiglu_mlp(x, wg, wu, wd, dy)
    eps = 1e-6
    args = [x, wg, wu, wd]

    def f(k, idx, delta):
        a = [m.copy() for m in args]
        a[k][idx] += delta
        return float((oracle.swiglu_mlp(*a) * dy).sum())

    for k, grad, idx in [(0, dx, (1, 2)), (1, dwg, (3, 0)), (2, dwu, (4, 3)), (3, dwd, (2, 1))]:
        fd = (f(k, idx, eps) - f(k, idx, -eps)) / (2 * eps)
        assert grad[idx] == pytest.approx(fd, abs=1e-7)


def test_swiglu_mlp_rows_are_independent():
    """The property TiledMLP relies on: a shard of rows gives the same rows
    as the whole sequence."""
    x, wg, wu, wd, dy = mlp_inputs(10, 6, 9, seed=4)
    y = oracle.swiglu_mlp(x, wg, wu, wd)
    np.testing.assert_array_equal(oracle.swiglu_mlp(x[3:7], wg, wu, wd), y[3:7])


def test_logits_loss_magnitudes_match_torch_absolute_sums():
    """The rounding-bound magnitudes of the loss: zmag_i = max_v sum_k
    |h_ik w_vk|, dh_mag = |G| |W|, dw_mag = |G|^T |H|, with G the gradient of
    s * loss_sum with respect to the logits, from torch's own cross-entropy
    and autograd (fp64)."""
    T, d, V, s = 11, 6, 17, 0.3
    h, w, labels = lm_inputs(T, d, V, seed=77, ignore_every=3)
    *_, mags = oracle.logits_loss(h, w, labels, s, magnitude=True)
    ht, wt = torch.tensor(h), torch.tensor(w)
    z = (ht @ wt.T).detach().requires_grad_(True)
    rows = torch.nn.functional.cross_entropy(z, torch.tensor(labels),
                                             ignore_index=oracle.IGNORE_INDEX, reduction="none")
    (s * rows.sum()).backward()
    g_abs = z.grad.abs()
    want_zmag = (ht.abs()[:, None, :] * wt.abs()[None, :, :]).sum(-1).max(-1).values
    np.testing.assert_allclose(mags["zmag"], want_zmag.numpy(), rtol=1e-13)
    np.testing.assert_allclose(mags["dh"], (g_abs @ wt.abs()).numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(mags["dw"], (g_abs.T @ ht.abs()).numpy(), rtol=1e-11, atol=1e-15)
    # and they bound the values they describe
    _, _, _, dh, dw = oracle.logits_loss(h, w, labels, s)
    assert np.all(np.abs(dh) <= mags["dh"] * (1 + 1e-12)) and np.all(np.abs(dw) <= mags["dw"] * (1 + 1e-12))


def test_swiglu_mlp_magnitudes_match_torch_absolute_sums():
    """The rounding-bound magnitudes of the MLP: y_mag = |a| |Wd|^T,
    dx_mag = |dg| |Wg| + |du| |Wu|, dwg_mag = |dg|^T |x|, dwu_mag = |du|^T |x|,
    dwd_mag = |dy|^T |a|, with a, dg and du from torch autograd (fp64)."""
    T, d, I = 7, 5, 9
    x, wg, wu, wd, dy = mlp_inputs(T, d, I, seed=31)
    *_, mags = oracle.swiglu_mlp(x, wg, wu, wd, dy, magnitude=True)
    xt, wgt, wut, wdt, dyt = (torch.tensor(a) for a in (x, wg, wu, wd, dy))
    g = (xt @ wgt.T).requires_grad_(True)
    u = (xt @ wut.T).requires_grad_(True)
    a = torch.nn.functional.silu(g) * u
    (a @ wdt.T).backward(dyt)
    dg, du, aa = g.grad.abs(), u.grad.abs(), a.detach().abs()
    want = {"y": aa @ wdt.abs().T, "dx": dg @ wgt.abs() + du @ wut.abs(), "dwg": dg.T @ xt.abs(),
            "dwu": du.T @ xt.abs(), "dwd": dyt.abs().T @ aa}
    for name, ref in want.items():
        np.testing.assert_allclose(mags[name], ref.numpy(), rtol=1e-11, atol=1e-15, err_msg=name)
    y_only = oracle.swiglu_mlp(x, wg, wu, wd, magnitude=True)
    np.testing.assert_allclose(y_only[1]["y"], want["y"].numpy(), rtol=1e-11, atol=1e-15)
