"""The language-model loss (lm_head GEMM + cross-entropy + gradients, logits
formed one shard of rows at a time) against the oracle, element by element.

Tolerances follow from the arithmetic (bf16 inputs are exact in fp32
products; logits, the row statistics and the label logit stay fp32; each G
element carries two bf16 roundings, of exp(z - tile max) and of G itself,
so |dG| <= (2^-8 + 2^-20) |G|; dh is rounded to bf16, dw stays fp32), with
the oracle's magnitudes zmag_i = max_v sum_k |h_ik w_vk|, |G| |W| and
|G|^T |H|, each bar twice the bound:
  loss_i : 2 d 2^-24 zmag_i + 1e-5 (1 + |loss_i|)
  dh     : 2^-7 (|G||W|) + 2^-8 |dh|
  dw     : 2^-7 (|G|^T|H|)
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import ensure_library, to_device

pytestmark = pytest.mark.gpu

W_SCALE = 2.0   # lm_head weight std = W_SCALE / sqrt(d): logits of std ~2


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_library()


def inputs(seed, T, d, V, ignore_percent):
    h = synth.normal(seed, synth.STREAM_HIDDEN, (T, d), "bf16")
    w = synth.normal(seed, synth.STREAM_LM_HEAD, (V, d), "bf16", scale=W_SCALE / np.sqrt(d))
    labels = synth.lm_labels(seed, T, V, ignore_percent)
    return h, w, labels


def run_gpu(h_bits, w_bits, labels, s, shard):
    import torch
    import ulysses_sp_attention_amd as uly
    T, d = h_bits.shape
    V = w_bits.shape[0]
    h = to_device(h_bits, "bf16")
    w = to_device(w_bits, "bf16")
    lab = torch.tensor(labels, dtype=torch.int64, device="cuda")
    rows = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    total = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    good = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    dh = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((V, d), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = uly.ulysses_logits_loss_workspace_size(max(min(shard, T), 1), V)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    uly.ulysses_logits_loss(h, w, lab, rows, total, good, dh, dw, ws, s, shard)
    torch.cuda.synchronize()
    return (rows.cpu().numpy().astype(np.float64), float(total.item()), int(good.item()),
            dh.float().cpu().numpy().astype(np.float64), dw.cpu().numpy().astype(np.float64))


def check(got, ref, mags, d):
    rows, total, good, dh, dw = got
    r_rows, r_total, r_good, r_dh, r_dw = ref
    tol_rows = 2 * d * 2.0 ** -24 * mags["zmag"] + 1e-5 * (1 + np.abs(r_rows))
    assert np.all(np.abs(rows - r_rows) <= tol_rows), np.max(np.abs(rows - r_rows) - tol_rows)
    assert good == r_good
    assert abs(total - r_total) <= tol_rows.sum() + 1e-6 * abs(r_total)
    tol_dh = 2.0 ** -7 * mags["dh"] + 2.0 ** -8 * np.abs(r_dh)
    assert np.all(np.abs(dh - r_dh) <= tol_dh), np.max(np.abs(dh - r_dh) - tol_dh)
    tol_dw = 2.0 ** -7 * mags["dw"]
    assert np.all(np.abs(dw - r_dw) <= tol_dw), np.max(np.abs(dw - r_dw) - tol_dw)


CASES = [
    # T, d, V, shard, grad_scale, ignore %
    (100, 64, 1000, 32, 1.0 / 90, 10),     # ragged last shard, V % 4 == 0 (vector rows)
    (37, 128, 997, 16, 1.0, 20),           # V % 4 != 0 (scalar rows), ragged
    (64, 256, 4100, 64, 0.01, 0),          # one shard, every token kept
    (130, 64, 515, 200, 0.5, 30),          # shard larger than T
    (9, 32, 3, 2, 1.0, 10),                # tiny vocabulary
]


@pytest.mark.parametrize("T,d,V,shard,s,ign", CASES)
def test_logits_loss_matches_oracle(T, d, V, shard, s, ign):
    seed = 7000 + T + V
    h, w, labels = inputs(seed, T, d, V, ign)
    ref = oracle.logits_loss(synth.to_f64(h, "bf16"), synth.to_f64(w, "bf16"), labels, s,
                             magnitude=True)
    got = run_gpu(h, w, labels, s, shard)
    check(got, ref[:5], ref[5], d)


def test_logits_loss_all_ignored():
    T, d, V = 50, 64, 516
    h, w, _ = inputs(11, T, d, V, 0)
    labels = np.full(T, synth.IGNORE_INDEX, dtype=np.int64)
    rows, total, good, dh, dw = run_gpu(h, w, labels, 1.0, 16)
    assert good == 0 and total == 0.0
    assert not rows.any() and not dh.any() and not dw.any()


def test_logits_loss_empty_input_zeroes_dw():
    rows, total, good, dh, dw = run_gpu(np.zeros((0, 64), np.uint16),
                                        synth.normal(3, synth.STREAM_LM_HEAD, (40, 64), "bf16"),
                                        np.zeros(0, np.int64), 1.0, 8)
    assert total == 0.0 and good == 0 and not dw.any()


def test_logits_loss_out_of_range_label_gives_nan_row_only_there():
    T, d, V = 20, 64, 100
    h, w, labels = inputs(13, T, d, V, 0)
    labels[5] = V            # neither a class nor the ignore index
    rows, _, _, dh, _ = run_gpu(h, w, labels, 1.0, 8)
    assert np.isnan(rows[5]) and np.all(np.isnan(dh[5]))
    keep = np.arange(T) != 5
    ref = oracle.logits_loss(synth.to_f64(h, "bf16")[keep], synth.to_f64(w, "bf16"),
                             labels[keep], magnitude=True)
    tol = 2 * d * 2.0 ** -24 * ref[5]["zmag"] + 1e-5 * (1 + np.abs(ref[0]))
    assert np.all(np.abs(rows[keep] - ref[0]) <= tol)


def test_logits_loss_is_reproducible():
    h, w, labels = inputs(17, 200, 128, 2048, 10)
    a = run_gpu(h, w, labels, 0.1, 64)
    b = run_gpu(h, w, labels, 0.1, 64)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x), np.asarray(y), equal_nan=True)


def test_logits_loss_full_size_llama8b_lm_head_sampled():
    """The Llama-8B lm_head (d = 4096, V = 128256) over one rank's 16384
    tokens, 4096 rows of logits at a time: sampled token rows of the loss and
    dh against the oracle on those rows (row i depends on h_i and W only),
    the kept-token count exactly, and the zero column sum of dW."""
    import torch
    import ulysses_sp_attention_amd as uly
    T, d, V, shard, seed = 16384, 4096, 128256, 4096, 4321
    h_bits = synth.normal(seed, synth.STREAM_HIDDEN, (T, d), "bf16")
    w_bits = synth.normal(seed, synth.STREAM_LM_HEAD, (V, d), "bf16", scale=W_SCALE / np.sqrt(d))
    labels = synth.lm_labels(seed, T, V, 10)
    h = to_device(h_bits, "bf16")
    w = to_device(w_bits, "bf16")
    lab = torch.tensor(labels, device="cuda")
    rows = torch.empty(T, dtype=torch.float32, device="cuda")
    total = torch.empty(1, dtype=torch.float32, device="cuda")
    good = torch.empty(1, dtype=torch.int64, device="cuda")
    dh = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((V, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(uly.ulysses_logits_loss_workspace_size(shard, V), dtype=torch.uint8,
                     device="cuda")
    s = 1.0 / max(int((labels != synth.IGNORE_INDEX).sum()), 1)
    uly.ulysses_logits_loss(h, w, lab, rows, total, good, dh, dw, ws, s, shard)
    torch.cuda.synchronize()
    assert int(good.item()) == int((labels != synth.IGNORE_INDEX).sum())
    # sampled rows: first, last, both sides of every shard boundary, one ignored token
    sample = sorted({0, T - 1, 4095, 4096, 8191, 8192, 12287, 12288,
                     int(np.nonzero(labels == synth.IGNORE_INDEX)[0][0])})
    ref = oracle.logits_loss(synth.to_f64(h_bits[sample], "bf16"), synth.to_f64(w_bits, "bf16"),
                             labels[sample], s, magnitude=True)
    r_rows, _, _, r_dh, _, mags = ref
    g_rows = rows.cpu().numpy()[sample].astype(np.float64)
    tol = 2 * d * 2.0 ** -24 * mags["zmag"] + 1e-5 * (1 + np.abs(r_rows))
    assert np.all(np.abs(g_rows - r_rows) <= tol)
    g_dh = dh.float().cpu().numpy()[sample].astype(np.float64)
    assert np.all(np.abs(g_dh - r_dh) <= 2.0 ** -7 * mags["dh"] + 2.0 ** -8 * np.abs(r_dh))
    # every row of G sums to zero, so sum_v dW_v = 0 up to rounding: the two
    # bf16 roundings of each G element (exp(z - tile max), then G) move a
    # row's sum by at most 2^-8 sum_v |G_iv| <= 2^-7 s; the fp32 GEMM sums
    # (4096 rows per shard) add at most 2^-12 * 2 s per row; the fp32
    # softmax's own sum error is below 2^-20 s: in all below 2^-6 s per row
    col = dw.double().sum(dim=0).cpu().numpy()
    bound = 2.0 ** -6 * s * h.double().abs().sum(dim=0).cpu().numpy()
    assert np.all(np.abs(col) <= bound)
    assert np.isfinite(float(total.item()))


def test_logits_loss_from_two_host_threads_at_once():
    """The call keeps no state between calls: two host threads calling at
    the same time on their own streams get the same bits as one call alone."""
    import threading
    import torch
    import ulysses_sp_attention_amd as uly
    T, d, V, shard = 96, 128, 3000, 32
    h_bits, w_bits, labels = inputs(23, T, d, V, 10)
    alone = run_gpu(h_bits, w_bits, labels, 0.5, shard)
    h = to_device(h_bits, "bf16")
    w = to_device(w_bits, "bf16")
    lab = torch.tensor(labels, device="cuda")
    outs, errors = [], []

    def worker():
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                rows = torch.empty(T, device="cuda")
                total = torch.empty(1, device="cuda")
                good = torch.empty(1, dtype=torch.int64, device="cuda")
                dh = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
                dw = torch.empty((V, d), device="cuda")
                ws = torch.empty(uly.ulysses_logits_loss_workspace_size(shard, V),
                                 dtype=torch.uint8, device="cuda")
                for _ in range(3):
                    uly.ulysses_logits_loss(h, w, lab, rows, total, good, dh, dw, ws, 0.5, shard)
            stream.synchronize()
            outs.append((rows.cpu().numpy().astype(np.float64), float(total.item()),
                         int(good.item()), dh.float().cpu().numpy().astype(np.float64),
                         dw.cpu().numpy().astype(np.float64)))
        except Exception as e:   # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=worker) for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert len(outs) == 2
    for got in outs:
        for x, y in zip(got, alone):
            assert np.array_equal(np.asarray(x), np.asarray(y))
