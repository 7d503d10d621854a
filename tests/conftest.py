import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import context_ring_attention_amd as cra
    cra.load()          # raises if libcpattn.so is not built
    return cra


def pytest_terminal_summary(terminalreporter):
    """The worst achieved errors against the oracle (forward and gradients), beside their bounds."""
    try:
        import parity_util
    except ImportError:
        return
    rec = parity_util.RECORD
    grad = parity_util.GRAD_RECORD
    if not rec and not grad:
        return
    tol = {"bf16": (parity_util.BF16_MAX_ABS, parity_util.BF16_REL_L2, parity_util.BF16_LSE_ABS),
           "fp32": (parity_util.F32_MAX_ABS, parity_util.F32_REL_L2, parity_util.F32_LSE_ABS)}
    tr = terminalreporter
    tr.section("parity margins against the oracle (achieved / bound)")
    for dt in ("bf16", "fp32"):
        rows = [r for r in rec if r[1] == dt]
        if not rows:
            continue
        t = tol[dt]
        for k, name in ((2, "O max-abs"), (3, "O rel-L2"), (4, "LSE abs")):
            worst = max(rows, key=lambda r: r[k])
            tr.write_line(f"{dt} {name}: worst {worst[k]:.3e} (bound {t[k - 2]:.0e}) in "
                          f"'{worst[0]}' over {len(rows)} checks")
    if grad:
        for k, name, bound in ((1, "rel-L2", "5e-03"), (2, "max-abs / max |ref|", "1e-02")):
            worst = max(grad, key=lambda r: r[k])
            tr.write_line(f"bf16 gradient {name}: worst {worst[k]:.3e} (bound {bound}) in "
                          f"'{worst[0]}' over {len(grad)} checks")
