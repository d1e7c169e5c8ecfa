"""The oracle's report scripts at reduced sizes: the per-layer logit-MAE comparison of Block-GTQ and
uniform widths (abstract), and the value-rotation reconstruction error (QWC summary, Results)."""
import io

import numpy as np

import synth
from oracle import report_logit_mae, report_value_rotation


def test_logit_mae_report_small():
    """Direction of the abstract's per-layer comparison on three synthetic layers, both budgets:
    Block-GTQ widths win every layer (soft check: the synthetic heads carry outlier blocks)."""
    buf = io.StringIO()
    s = report_logit_mae.report(layers=3, n_tokens=256, n_pos=2, out=buf)
    for U, r in s.items():
        assert r["won"] == r["layers"] == 3, (U, r)
        assert 0.0 < r["red_min"] <= r["red_med"] <= r["red_max"] < 1.0
    assert "| K3 (192 units) | 3/3 |" in buf.getvalue()


def test_value_rotation_is_neutral_on_iid_rows_and_helps_outlier_channels():
    """An orthogonal rotation maps iid Gaussian rows to iid Gaussian rows: the reconstruction error
    stays within a few percent.  Rows with two large channels spread them over the group and lose
    much less under the rotation (codebook and affine)."""
    w = synth.WORKLOADS[2]
    for mode, bits in (("codebook", 3), ("affine", 2)):
        r = report_value_rotation.measure(w, mode, bits, 512, outliers=False, heads=((0, 0),))
        assert abs(r[True][0] / r[False][0] - 1.0) < 0.05, (mode, r)
        ro = report_value_rotation.measure(w, mode, bits, 512, outliers=True, heads=((0, 0),))
        assert ro[True][0] < 0.5 * ro[False][0], (mode, ro)


def test_value_rotation_reconstruction_round_trips_at_high_width():
    """With 4-bit affine groups the rotated path reconstructs the rows in the original space
    (rotated back exactly), within the quantizer's error."""
    v = np.random.default_rng(0).standard_normal((64, 128)).astype(np.float32)
    s = report_value_rotation._signs(1)
    vh = report_value_rotation.reconstruct(v, "affine", 4, s)
    assert np.sqrt(np.mean((vh - v) ** 2)) < 0.15
