"""Host-side checks of the seeded input generator (no BitDelta arithmetic)."""
import numpy as np

from tenant_serving_amd import synth as S


def test_same_seed_same_bytes_and_row_slices_agree():
    w = S.workload(3)
    a = S.host_wbase(w, 2, rows=[5, 100, 4095])
    b = S.host_wbase(w, 2, rows=[5, 100, 4095])
    assert np.array_equal(a, b)
    full = S.host_normal(S.key(w, S.KIND_WBASE, 0, 2), w.dtype, 8, w.matrices[2].d_in, 0.02)
    assert np.array_equal(full[5:6], S.host_wbase(w, 2, rows=[5]))
    f1 = S.host_wfine(w, 2, 7, rows=[5, 6])
    f2 = S.host_wfine(w, 2, 7, rows=[6])
    assert np.array_equal(f1[1], f2[0])
    assert not np.array_equal(S.host_wfine(w, 2, 8, rows=[6]), f2)


def test_distributions_have_the_stated_moments():
    w = S.workload(2)
    wb = S.as_f32(S.host_wbase(w, 0, rows=range(64)), w.dtype).astype(np.float64)
    assert abs(wb.std() - 0.02) < 5e-4 and abs(wb.mean()) < 5e-4
    wf = S.as_f32(S.host_wfine(w, 0, 1, rows=range(64)), w.dtype).astype(np.float64)
    d = wf - wb
    assert abs(np.abs(d).mean() - 5e-4) < 3e-5   # Laplace(0,b): E|d| = b (before bf16 rounding)
    assert 0.05 < (d == 0).mean() < 0.12           # bf16 rounding zeroes a share of deltas
    x = S.as_f32(S.host_x(w, 0), w.dtype).astype(np.float64)
    assert x.shape == (16, 4096) and abs(x.std() - 1) < 0.02


def test_outliers_are_injected_at_the_stated_rate():
    w = S.workload(3)
    wb = S.host_wbase(w, 0, rows=range(256))
    wf = S.host_wfine(w, 0, 0, rows=range(256), wbase=wb)
    d = S.as_f32(wf, w.dtype).astype(np.float64) - S.as_f32(wb, w.dtype)
    big = np.abs(d) > 20 * w.b
    assert 0.0006 < big.mean() < 0.0014
    assert np.allclose(np.abs(d[big]), w.outlier_mag, rtol=0.02)


def test_user_id_recipes():
    ids2 = S.user_ids(S.workload(2))
    assert sorted(ids2.tolist()) == list(range(16))
    ids3 = S.user_ids(S.workload(3))
    assert len(ids3) == 256 and ids3.min() >= 0 and ids3.max() < 64
    w4 = S.workload(4)
    ids4 = S.user_ids(w4)
    assert len(ids4) == 1144
    for c in range(8):
        assert len(set(ids4[128 * c:128 * (c + 1)].tolist())) == 1
    ids5 = S.user_ids(S.workload(5))
    counts = np.bincount(ids5, minlength=128)
    assert len(ids5) == 512 and counts[0] == counts.max() and counts[0] > 60  # Zipf head
    assert np.array_equal(ids5, S.user_ids(S.workload(5)))


def test_workload_shapes():
    w5 = S.workload(5)
    assert len(w5.matrices) == 224
    n = sum(m.d_out * m.d_in for m in w5.matrices)
    assert n * 2 == 13_958_643_712  # 13.96 GB of bf16 base weights
