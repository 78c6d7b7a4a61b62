import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: generates full-size layers")


def weights_kwargs(weights):
    """The weight arrays of a synth.Weights as keyword arguments."""
    return {a: getattr(weights, a) for a in weights.ARRAYS}


def assert_out_close(got, ref, rel=2e-2, what="out"):
    """Element-wise |g - r| <= rel * max(|r|, rms(r)) over the whole output."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * np.maximum(np.abs(ref), rms)
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {got.size} elements outside tolerance; worst at {i}: "
            f"got {got[i]!r} ref {ref[i]!r} (rms {rms:.3g}); max|g-r|/max|r| = "
            f"{float(err.max() / max(np.abs(ref).max(), 1e-300)):.3g}")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
