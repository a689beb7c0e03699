"""The seeded input generators: shapes, determinism and the structure the
workloads call for (outlier counts, Zipf top-8 routing, 128-padded groups)."""
import numpy as np

import synthetic


def test_bf16_roundtrip_and_rounding():
    x = np.array([1.0, -2.5, 1.00390625, 1.01171875, 3.0e38], np.float32)
    b = synthetic.bf16_from_f32(x)
    back = synthetic.bf16_to_f32(b)
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[2] == 1.0                        # 1 + 2^-8 is a tie -> even
    assert back[3] == np.float32(1.015625)       # 1 + 3*2^-8 is a tie -> even (up)


def test_tiny_linear_outliers():
    x, w = synthetic.tiny_linear()
    assert x.shape == (256, 512) and w.shape == (256, 512) and x.dtype == np.float32
    base = synthetic.normal_f32((256, 512), 101)
    changed = np.count_nonzero(x != base)
    assert changed == round(0.001 * x.size)
    x2, _ = synthetic.tiny_linear()
    assert np.array_equal(x, x2)


def test_heavy_tail():
    base = synthetic.normal_f32((64, 1024), 5, 1e-3)
    y = synthetic.heavy_tail_f32(base, 0.001, 6)
    ratio = y[y != base] / base[y != base]
    assert ratio.size == round(0.001 * base.size)
    assert np.all((ratio >= 10 * 0.999) & (ratio <= 1000 * 1.001))


def test_moe_routing_structure():
    m = synthetic.moe(T=1024, H=256, G=16, I=128, with_weights=False)
    assert m.counts.sum() == 1024 * 8
    assert np.all(np.diff(m.offsets) % 128 == 0)
    assert np.all(np.diff(m.offsets) >= m.counts)
    assert m.offsets[0] == 0 and m.offsets[-1] == m.a_gate_up.shape[0]
    real = m.token_index >= 0
    assert np.all(m.a_gate_up[~real] == 0) and np.all(m.a_down[~real] == 0)
    assert np.array_equal(m.a_gate_up[real], m.x[m.token_index[real]])
    # each token appears in exactly 8 distinct groups
    assert np.all(np.bincount(m.token_index[real], minlength=1024) == 8)
    # Zipf popularity: expert 0 is the most chosen
    assert m.counts[0] == m.counts.max()
    for e in range(16):
        toks = m.token_index[m.offsets[e]:m.offsets[e] + m.counts[e]]
        assert np.all(np.diff(toks) > 0)


def test_long_k_row_magnitudes():
    x, w = synthetic.long_k(M=64, N=128, K=256)
    xf = synthetic.bf16_to_f32(x)
    rms = np.sqrt((xf.astype(np.float64) ** 2).mean(axis=1))
    assert rms.max() / rms.min() > 10        # log-normal row magnitudes span decades
    assert w.shape == (128, 256)
