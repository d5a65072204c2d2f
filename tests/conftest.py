import json
import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name: str):
    with open(GOLDEN / name, encoding="utf-8") as f:
        return json.load(f)


@pytest.fixture(scope="session")
def hip():
    """The HIP binding with a usable GPU, or skip (GPU tests only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import dspark_verify_scheduling_amd as dv

    dv.load()  # raises if the built library is missing
    return dv


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run before touching the GPU
    os.environ.setdefault("PYTHONUNBUFFERED", "1")
