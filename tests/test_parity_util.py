"""The per-row gate of the full-size parity tests catches a single wrong row
that the tensor-wide rel-L2 lets through (CPU, no GPU needed)."""
import numpy as np

from parity_util import rel_l2, max_row_err, ROW_MULT, TOL


def test_one_bad_row_is_caught():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((16384, 64))
    noisy = ref * (1 + 2.0 ** -9 * rng.standard_normal(ref.shape))  # bf16-like rounding
    tol_f, tol_b = TOL["bf16"]
    assert max_row_err(noisy, ref) < ROW_MULT * tol_f
    for bad in ("zero", "flip", "scale"):
        x = noisy.copy()
        if bad == "zero":
            x[16383] = 0
        elif bad == "flip":
            x[7] = -x[7]
        else:
            x[100] *= 1.2
        assert rel_l2(x, ref) < tol_b  # invisible to the tensor-wide figure
        assert max_row_err(x, ref) > ROW_MULT * tol_b


def test_masked_rows_must_be_zero():
    ref = np.ones((100, 8))
    ref[10] = 0.0                                   # a masked row
    x = ref.copy()
    assert max_row_err(x, ref) == 0.0
    x[10] = 0.5                                      # nonzero where the reference is zero
    assert max_row_err(x, ref) > 1.0
