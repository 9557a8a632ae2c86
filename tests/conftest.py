import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Build the in-tree libraries once if they are missing (a fresh checkout keeps no built
    files); a tree that has them is used as it is."""
    from decode_attention_sequence_paged_amd import build as pkg_build
    from dcp_inputs import HOST_LIB_PATH, SYNTH_LIB_PATH
    from dcp_inputs import build as inputs_build
    if not os.path.exists(pkg_build.LIB_PATH):
        pkg_build.build_lib()
    if not (os.path.exists(HOST_LIB_PATH) and os.path.exists(SYNTH_LIB_PATH)):
        inputs_build.build_all()


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, where no GPU is visible (e.g. CPU-only runs).
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
