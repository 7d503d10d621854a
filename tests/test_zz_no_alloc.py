"""cpattn_fwd_chunks_noalloc (plan in the library's static device scratch) against
cpattn_fwd_chunks (plan in a caller workspace), through the C ABI.

Calls in a row on one stream, the second with a smaller input, each compared with the
workspace entry point's output on the same inputs (bit for bit: same kernels, same plan) and
with the oracle to the parity bar; a plan beyond the static scratch is refused.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import share_ref
from parity_util import check, dev, host

pytestmark = pytest.mark.gpu


def _run_both(cra, g, dtype):
    import torch
    q = dev(g.q, dtype)
    ks = [dev(c.k, dtype) for c in g.chunks]
    vs = [dev(c.v, dtype) for c in g.chunks]
    args = (q, ks, vs, g.cu_q, [c.cu_k for c in g.chunks], g.q_off, [c.k_off for c in g.chunks])
    o_ws, l_ws = cra.cpattn_fwd_chunks(*args)
    tq, hq, d = q.shape
    o_na = torch.full((tq, hq, d), float("nan"), device="cuda")
    l_na = torch.full((hq, tq), float("nan"), device="cuda")
    cra.cpattn_fwd_chunks_noalloc(*args, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


def test_noalloc_equals_workspace_entry_point_on_two_calls(gpu_lib):
    import torch
    # first call: the CP4 share of a 16,384-token pack (4 chunks); second: a smaller share
    # (2 chunks of a short pack) that reuses the same scratch
    big = wl.make("cp4_share", 0).groups[0]
    rng = np.random.default_rng(42)
    small = wl._even_split_group(rng, [300, 77, 5], 2, 32, 8, 128, "bf16", 1)
    # third: 150 short sequences (metadata too large for the device planner: the plan is built
    # in the entry point's static host buffer and copied into the static device scratch)
    many = wl._even_split_group(rng, [int(x) for x in rng.integers(1, 20, size=150)], 2, 4, 2, 64,
                                "bf16", 1)
    for name, g in (("cp4 share", big), ("small share", small), ("many sequences", many)):
        o_ws, l_ws, o_na, l_na = _run_both(gpu_lib, g, "bfloat16")
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), name
        rows = np.arange(int(g.cu_q[-1])) if name != "cp4 share" else \
            np.unique(np.linspace(0, int(g.cu_q[-1]) - 1, 300).astype(np.int64))
        check(host(o_na)[rows], host(l_na)[:, rows], *share_ref(g, rows=rows), "bf16",
              f"no-alloc {name}")


def test_noalloc_refuses_a_plan_beyond_its_scratch(gpu_lib):
    import torch
    # 16 chunks x 8,193 query tiles of 32 tokens = 131,088 plan records > 131,072
    tq, nch = 8193 * 32, 16
    q = torch.zeros((tq, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64), dtype=torch.bfloat16, device="cuda")
    cu_q = np.array([0, tq], np.int32)
    cu_k = [np.array([0, 1], np.int32)] * nch
    with pytest.raises(gpu_lib.CpattnError) as e:
        gpu_lib.cpattn_fwd_chunks_noalloc(q, [k] * nch, [k] * nch, cu_q, cu_k)
    assert e.value.status == 2 and "static scratch" in str(e.value)
    # the library still works afterwards
    g = wl.make("pack", 1).groups[0]
    o_ws, l_ws, o_na, l_na = _run_both(gpu_lib, g, "bfloat16")
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
