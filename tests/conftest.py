import os
import sys
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# The tests drive the library's GLASS_AMD_* placement and launch-shape
# switches; the library honours them only in a process that set this before
# its first call.
os.environ.setdefault("GLASS_AMD_TUNING", "1")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def read_golden(name):
    """Parse a ``key value value ...`` fixture; '#' starts a comment line.
    Values are returned as Fractions (exact)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [Fraction(v) for v in vals]
    return out


def frac_array(vals):
    return np.array([float(v) for v in vals], dtype=np.float64)


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0.  Skips where there is no GPU; where there is
    one, a missing or unloadable library is an error, never a silent
    fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import block_tridiagonal_pcg_bdmv_amd as glass
    glass.load()  # raises if the library is missing
    return glass
