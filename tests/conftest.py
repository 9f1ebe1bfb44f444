import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large full-size case")


# GPU test modules run bottom-up: the building blocks (scores, top-k, pool step) before the
# whole decode step, then the prefill indexer, then what is built on top (steps in a row, the
# inter-query prefetch, several layers, the scoring launch with a host-gather wave), and the
# full-size stress step last, so that under -x the first failure names the lowest broken piece
# and hides no result below it.  Other modules keep their place before these; test_zz_* stay
# last.
BOTTOM_UP = ("test_gpu_scores.py", "test_gpu_topk.py", "test_gpu_pool.py", "test_gpu_decode.py",
             "test_gpu_prefill.py", "test_gpu_multistep.py", "test_gpu_interquery.py",
             "test_gpu_layers.py", "test_gpu_fused.py", "test_gpu_stress.py")


def _order(item):
    name = os.path.basename(str(item.fspath))
    if name.startswith("test_zz_"):
        return len(BOTTOM_UP) + 1
    return BOTTOM_UP.index(name) + 1 if name in BOTTOM_UP else 0


def pytest_collection_modifyitems(config, items):
    items.sort(key=_order)                   # stable: the order inside each group is kept
    # gpu tests cannot run without a device: skip them cleanly when none is visible
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
