"""The seeded input generators: shapes, determinism and the planted structure."""
import math

import torch

import synthetic as syn


def test_generators_are_deterministic():
    a = syn.c2(rows=64, vocab=512, canvas_len=16)
    b = syn.c2(rows=64, vocab=512, canvas_len=16)
    assert torch.equal(a.logits, b.logits) and torch.equal(a.temps, b.temps)


def test_c1_shape_and_temps():
    w = syn.c1(rows=64, vocab=1024)
    assert w.logits.shape == (64, 1024) and w.canvas_len == 32
    assert w.temps.tolist() == [1.0, 0.0] and w.probs_dtype == torch.bfloat16


def test_c2_peaks_and_temps():
    w = syn.c2(rows=256, vocab=4096, canvas_len=16)
    peaked = w.special_rows["peaked"]
    assert len(peaked) == 256 // 8
    assert float(w.logits[peaked].max(dim=1).values.min()) > 10.0
    assert sorted(set(w.temps.tolist())) == sorted({0.0, float(torch.tensor(0.7)), 1.0})


def test_c3_adversarial_rows():
    w = syn.c3(rows=200, vocab=2048, n_adv_per_kind=4, boundary=512)
    x = w.logits
    for r in w.special_rows["all_equal"].tolist():
        assert torch.all(x[r] == x[r, 0])
    for r in w.special_rows["dup_max"].tolist():
        assert int((x[r] == x[r].max()).sum()) >= 2
    for r in w.special_rows["neg_inf_span"].tolist():
        n = int(torch.isinf(x[r]).sum())
        assert 0.09 * x.shape[1] <= n < x.shape[1]
    for r in w.special_rows["huge"].tolist():
        t = float(w.temps[r])
        assert torch.all(torch.isfinite(x[r] / t))
        assert float(x[r].abs().min()) >= 0.49 * 3.4e38 * min(t, 1.0)
    for r in w.special_rows["subnormal"].tolist():
        tiny = (x[r] != 0) & (x[r].abs() < 2.0 ** -126)
        assert int(tiny.sum()) > 0
    assert float(w.temps.min()) >= 0.1 and float(w.temps.max()) <= 1.5


def test_c4_keep_and_ties():
    w = syn.c4(rows=64, vocab=2048, canvas_len=4, K=20)
    assert int(w.keep_mask.sum()) == 8
    kept_t = set(w.temps[w.keep_mask.bool()].tolist())
    assert kept_t == {0.0, 1.0}
    for r in w.special_rows["kth_tie"].tolist():
        v = torch.sort(w.logits[r], descending=True).values
        assert v[19] == v[20]


def test_c5_stride_and_mix():
    w = syn.c5(rows=64, vocab=1024, canvas_len=8, pad=128)
    assert w.logits.stride(0) == 1024 + 128 and w.logits.stride(1) == 1
    assert len(w.special_rows["zipf"]) == 32
    z = int(w.special_rows["zipf"][0])
    v = torch.sort(w.logits[z], descending=True).values
    # rank-k value close to -1.1 ln k
    assert abs(float(v[99]) + 1.1 * math.log(100)) < 0.5
    assert int((w.temps == 0).sum()) == 2 and float(w.temps.max()) <= 1.5
