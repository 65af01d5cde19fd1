import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Tests marked gpu are skipped when no GPU is visible, so that "-m 'not gpu'" and a plain
    # run on a CPU-only machine behave the same; where a GPU is visible they run.
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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # boundary flips counted by every GPU-vs-oracle check of the session (tests/parity.py)
    parity = sys.modules.get("parity")
    log = getattr(parity, "FLIP_LOG", None)
    if not log:
        return
    tr = terminalreporter
    tr.write_sep("-", "boundary flips, GPU vs oracle (accept / draw / top-p)")
    total = {"accept": 0, "draw": 0, "topp": 0}
    seqs = 0
    for label, flips, nseq in log:
        seqs += nseq
        for k in total:
            total[k] += flips[k]
        if any(flips.values()):
            tr.write_line(f"{label}: {flips} over {nseq} sequences")
    tr.write_line(f"{len(log)} checks, {seqs} sequences: accept {total['accept']}, "
                  f"draw {total['draw']}, topp {total['topp']}")
