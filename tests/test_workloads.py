"""The seeded input generator: bf16 rounding, exact counts, label law,
reproducibility."""
import numpy as np
import pytest
import torch

import workloads as WL


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 37,
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, -3e38, 65504.0,
                  1.00390625, 1.01171875], dtype=np.float32),
        # halfway cases in both directions
        np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32
                 ).view(np.float32),
    ])
    got = WL.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, want.view(np.uint16))
    back = WL.bf16_bits_to_f32(got)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16)
                          .float().numpy())


def test_small_workloads_shapes_counts_and_reproducibility():
    for w in WL.WORKLOADS[:2]:
        a = WL.make_inputs(w, 0)
        b = WL.make_inputs(w, 0)
        assert a.H.shape == (w.N, w.d) and a.W.shape == (w.V, w.d)
        assert np.array_equal(a.H, b.H) and np.array_equal(a.W, b.W)
        assert np.array_equal(a.labels, b.labels)
        assert (a.labels == -100).sum() == w.n_ignored
        ok = a.labels[a.labels != -100]
        assert ok.min() >= 0 and ok.max() < w.V
        c = WL.make_inputs(w, 1)
        assert not np.array_equal(a.H, c.H)
    tiny = WL.make_inputs(WL.WORKLOADS[0], 0)
    assert tiny.H.dtype == np.float32
    assert abs(tiny.W.std() - 0.02) < 0.002
    assert abs(tiny.H.std() - 1.0) < 0.05
    assert (tiny.labels == -100).sum() == 0


def test_stated_ignored_and_outlier_counts():
    assert [w.n_ignored for w in WL.WORKLOADS] == [0, 205, 328, 1311, 13107]
    assert WL.WORKLOADS[4].n_outliers == 1311


def test_outlier_rows_scaled_before_single_rounding():
    w = WL.custom(N=400, d=32, V=50, R=2, outlier_frac=0.05,
                  outlier_scale=20.0)
    a = WL.make_inputs(w, 0)
    assert a.outlier_rows.size == 20
    h = WL.bf16_bits_to_f32(a.H)
    norms = np.linalg.norm(h, axis=1)
    big = np.zeros(400, bool)
    big[a.outlier_rows] = True
    assert norms[big].min() > 5 * norms[~big].max() / 2
    # the same stream without outliers gives the other rows unchanged
    w0 = WL.custom(N=400, d=32, V=50, R=2)
    b = WL.make_inputs(w0, 0)
    assert np.array_equal(a.H[~big], b.H[~big])


def test_chunked_generation_equals_one_shot():
    rng1 = np.random.default_rng(5)
    rng2 = np.random.default_rng(5)
    a = WL._normal_matrix(rng1, 37, 11, 0.3, True, chunk_rows=5)
    b = WL._normal_matrix(rng2, 37, 11, 0.3, True, chunk_rows=1000)
    assert np.array_equal(a, b)


def test_zipf_head_frequencies():
    V, s, n = 5000, 1.1, 400000
    w = WL.custom(N=n, d=8, V=V, R=1, labels="zipf", zipf_s=s)
    _, _, rl, rp, ri, _ = WL._streams(3)
    lab = WL.make_labels(w, rl, rp, ri)
    _, _, _, rp2, _, _ = WL._streams(3)
    perm = rp2.permutation(V)
    k = np.arange(1, V + 1, dtype=float)
    pmf = k ** -s / np.sum(k ** -s)
    counts = np.bincount(lab, minlength=V)
    for rank in range(5):
        got = counts[perm[rank]] / n
        sd = np.sqrt(pmf[rank] * (1 - pmf[rank]) / n)
        assert abs(got - pmf[rank]) < 5 * sd
    assert counts.sum() == n


@pytest.mark.parametrize("i", [0, 1, 2, 3, 4])
def test_workload_table(i):
    w = WL.WORKLOADS[i]
    assert w.R <= w.V
    if w.dtype == "bf16":
        assert w.d % 8 == 0
    if i == 3:
        assert abs(w.w_std * np.sqrt(w.d) - 3.0) < 1e-12
