import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


_GPU_GATE = {}


def _gpu_gate_error():
    """Why GPU tests cannot run here (None when they can): a GPU test must
    run the HIP library, so it fails -- never skips -- when torch sees no GPU
    or libswz.so is not mapped into this process."""
    if "error" not in _GPU_GATE:
        err = None
        try:
            import torch

            import tiled_movement_amd as T

            if not torch.cuda.is_available():
                err = "torch sees no GPU"
            else:
                with open("/proc/self/maps") as f:
                    maps = f.read()
                if os.path.realpath(T.LIB_PATH) not in maps:
                    err = f"{T.LIB_PATH} is not mapped into the test process"
        except Exception as e:  # import failures included
            err = f"{type(e).__name__}: {e}"
        _GPU_GATE["error"] = err
    return _GPU_GATE["error"]


@pytest.fixture(autouse=True)
def _gpu_gate(request):
    if request.node.get_closest_marker("gpu") is not None:
        err = _gpu_gate_error()
        if err:
            pytest.fail(f"GPU test cannot run: {err}", pytrace=False)


def read_kv(name):
    """key=value fixture file -> dict of ints (comments start with #)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = int(v)
    return out


def read_rows(name):
    """Whitespace table fixture -> list of token lists (comments start with #)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows
