import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def load_hand_blocks():
    """Parse tests/golden/q4_0_hand_blocks.txt -> list of (name, x f32[32],
    d, bytes u8[18])."""
    out = []
    with open(os.path.join(GOLDEN, "q4_0_hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, spec, d, hexes = [p.strip() for p in line.split("|")]
            x = np.zeros(32, dtype=np.float32)
            if spec.startswith("ramp"):
                x = (np.arange(32) - 16).astype(np.float32)
            elif spec != "zeros":
                for kv in spec.split():
                    k, v = kv.split("=")
                    x[int(k)] = float(v)
            b = np.array([int(h, 16) for h in hexes.split()], dtype=np.uint8)
            out.append((name, x, float(d), b))
    return out


@pytest.fixture
def hand_blocks():
    return load_hand_blocks()
