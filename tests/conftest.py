import os
import sys

import pytest
import torch  # noqa: F401  (first: every HIP library in the process then binds to torch's runtime)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _need_build():
    libs = ["oracle/liboracle.so", "synth/libsynth_host.so", "synth/libsynth_gpu.so",
            "int4_quantized_expert_amd/libmoe.so"]
    return any(not os.path.exists(os.path.join(ROOT, p)) for p in libs)


if _need_build():
    import __graft_entry__  # noqa: E402

    __graft_entry__.build()
