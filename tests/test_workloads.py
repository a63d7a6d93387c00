"""Shape, seeding and padding checks of the synthetic score generators."""
import numpy as np

from exact_row_wise_sampled_amd import workloads as W


def test_tiny_shape_and_lengths():
    w = W.tiny()
    assert w.x.shape == (4, 8192) and w.k == 256
    assert list(w.ke) == [8192, 6000, 3000, 1024]
    assert w.score_bytes() == 4 * (8192 + 6000 + 3000 + 1024)


def test_deterministic_per_seed():
    a = W.decode(seed=2, m=6, n=4096, lo=1024)
    b = W.decode(seed=2, m=6, n=4096, lo=1024)
    c = W.decode(seed=3, m=6, n=4096, lo=1024)
    assert np.array_equal(a.x.view(np.uint32), b.x.view(np.uint32))
    assert np.array_equal(a.ke, b.ke)
    assert not np.array_equal(a.x.view(np.uint32), c.x.view(np.uint32))


def test_decode_lengths_and_score_model():
    w = W.decode(m=16, n=8192, lo=2048)
    assert w.ke.min() >= 2048 and w.ke.max() <= 8192
    for r in range(16):
        v = w.x[r, :w.ke[r]]
        assert np.isfinite(v).all() and (v >= 0).all()     # sum of w * relu(.)
        assert (v == 0).mean() < 0.02                       # all 8 heads negative: 1/256


def test_padding_is_garbage():
    w = W.decode(m=4, n=8192, lo=1024)
    r = int(np.argmin(w.ke))
    pad = w.x[r, w.ke[r]:]
    assert pad.size > 0
    assert np.isnan(pad).mean() > 0.2 and np.isposinf(pad).mean() > 0.2


def test_prefill_lengths():
    w = W.prefill(m=8, n=1024, first=1000)
    assert list(w.ke) == [min(1000 + r + 1, 1024) for r in range(8)]


def test_long_rows_have_spikes():
    w = W.long_rows(m=2, n=1 << 16)
    assert (w.ke == 1 << 16).all()
    for r in range(2):
        v = w.x[r].astype(np.float64)
        # spikes sit about 3 sigma above the bulk: the row's maximum is far out
        assert v.max() > v.mean() + 4 * v.std()


def test_adversarial_row_types():
    w = W.adversarial(m=16, n=8192, lo=4096)
    for r in range(16):
        v = w.x[r, :w.ke[r]]
        t = r % 4
        if t == 0:
            assert np.unique(v).size <= 64 and (v * 8 == np.round(v * 8)).all()
        elif t == 1:
            assert (np.diff(v) >= 0).all()
        elif t == 2:
            assert np.unique(v.view(np.uint32)).size == 1
        else:
            assert np.isneginf(v[~np.isposinf(v)]).mean() > 0.2
            assert (v.view(np.uint32) == 0x80000000).any()   # -0.0 present
