import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


def _oracle_stale():
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib):
        return True
    src_m = max(os.path.getmtime(os.path.join(ROOT, "oracle", f)) for f in ("oracle.c", "oracle.h"))
    return os.path.getmtime(lib) < src_m


def pytest_sessionstart(session):
    # The oracle is plain C; (re)build it when missing or older than its source.
    if _oracle_stale():
        from oracle import build
        build.build()
    # The HIP library is built ahead of time (__graft_entry__.build()). Only on
    # a machine without a GPU, where the suite checks host logic, is a missing
    # library built here; on a GPU machine a missing library must fail.
    lib = os.path.join(ROOT, "block_table_gather_amd", "libhp.so")
    if not os.path.exists(lib):
        import torch
        if not torch.cuda.is_available():
            import importlib.util
            spec = importlib.util.spec_from_file_location(
                "_hp_build", os.path.join(ROOT, "block_table_gather_amd", "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build()


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
