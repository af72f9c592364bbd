"""Shared pytest configuration.

Markers:
  gpu - needs an MI355X (gfx950) and the built HIP library; everything else
        runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libfp8bs.so")


@pytest.fixture(scope="session")
def big_layer():
    """Oracle-quantized X (4096 x 7168, outliers, seed 0) and W (18432 x 7168,
    N(0, 0.02), seed 1): the Fprop layer of the bench, shared by the GEMM and
    fused-kernel tests (quantizing W on the host takes a while)."""
    import synthetic as syn
    from oracle import quant
    xb = syn.activation_with_outliers(4096, 7168, seed=0)
    wb = syn.gaussian((18432, 7168), seed=1, std=0.02)
    Xq, sX = quant.quant_rows(xb)
    del xb
    Wq, sW = quant.quant_weight(wb)
    del wb
    return Xq, sX, Wq, sW


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; the test fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import fine_grained_fp8_amd as fp8
    fp8.load_library()  # raises if libfp8bs.so is not built
    return fp8


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the element classes of every GEMM tolerance check of the run
    (and write them as JSON to $FP8BS_TOLERANCE_RECORD when that is set)."""
    try:
        from tolerance import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", "GEMM tolerance classes (elements per check)")
    tr.write_line(f"{'check':44s} {'K':>6s} {'n':>9s} {'<=2ulp':>9s} {'fp32sum':>8s} "
                  f"{'trunc':>6s} {'fail':>5s} {'exact':>9s} {'normwise':>9s}")
    for r in RECORDS:
        tr.write_line(f"{r['label'][:44]:44s} {r['K']:6d} {r['n']:9d} {r['within_2ulp']:9d} "
                      f"{r['fp32_sum_bound']:8d} {r['truncation_bound']:6d} {r['failed']:5d} "
                      f"{r['exact_match']:9d} {r['norm_err']:9.2e}")
    path = os.environ.get("FP8BS_TOLERANCE_RECORD")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(RECORDS, f, indent=1)
