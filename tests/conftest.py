import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_exact(values):
    """Decimal literals (or "-0") -> bf16 bit patterns; asserts each is exactly representable."""
    out = []
    for v in values:
        f = np.float32(-0.0) if v == "-0" else np.float32(float(v))
        assert float(f) == (float(v) if v != "-0" else -0.0)
        u = int(np.array(f, dtype=np.float32).view(np.uint32))
        assert u & 0xFFFF == 0, f"{v} is not exactly representable in bf16"
        out.append(u >> 16)
    return np.array(out, dtype=np.uint16)


def hex_bytes(s):
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)
