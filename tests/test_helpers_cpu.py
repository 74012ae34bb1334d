"""The parity metric and the error report used by the GPU tests (CPU only)."""
import numpy as np

from tests.helpers import err_report, rel_err


def test_err_report_figures_on_a_worked_case():
    ref = np.array([3.0, -4.0, 0.0, 0.0])          # rms = sqrt(25/4) = 2.5, max |ref| = 4
    got = np.array([3.3, -4.0, 0.01, 0.0])
    rep = err_report(got, ref, block=3)            # blocks of 3 cross the array's end
    assert rep["n"] == 4 and abs(rep["rms"] - 2.5) < 1e-15
    # bar: max(0.3 / (3 + 2.5), 0.01 / 2.5) = 0.3 / 5.5
    assert abs(rep["bar"] - 0.3 / 5.5) < 1e-12
    assert abs(rep["bar"] - rel_err(got, ref)) < 1e-15
    # inf-norm: max |d| / max |ref| = 0.3 / 4
    assert abs(rep["inf"] - 0.3 / 4) < 1e-12
    # per element with a floor of 1e-3 rms = 0.0025: max(0.3 / 3, 0.01 / 0.0025) = 4
    assert abs(rep["floor"] - 4.0) < 1e-12


def test_err_report_nan_and_empty():
    rep = err_report(np.array([1.0, np.nan]), np.array([1.0, 2.0]))
    assert np.isnan(rep["bar"]) and np.isnan(rep["inf"]) and np.isnan(rep["floor"])
    assert err_report(np.zeros(0), np.zeros(0))["bar"] == 0.0
