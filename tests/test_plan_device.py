"""The device planner (the forward's plan built on the GPU from metadata passed by value)
against the host planner, and a device-planned forward captured into a graph and replayed.

The plan is deterministic: the device planner must reproduce the host planner's entries and
their longest-first order byte for byte, for every geometry, chunk count and causal mode.
"""
import numpy as np
import pytest

import workloads as wl
from parity_util import dev

pytestmark = pytest.mark.gpu


def _host_and_device(cra, cu_q, cu_ks, q_off, k_offs, **kw):
    host, info = cra.cpattn_plan_build_chunks(cu_q, cu_ks, q_off, k_offs, **kw)
    devp = cra.cpattn_plan_build_device(cu_q, cu_ks, q_off, k_offs, **kw)
    return host, devp


def _tile_tokens(cra, **kw):
    """Tokens per tile of the forward's geometry for these heads and head size."""
    cu = wl.cu_from_lengths([1])
    return cra.cpattn_plan_build_chunks(cu, [cu], None, None, **kw)[1]["tokens_per_tile"]


@pytest.mark.parametrize("dtype,hq,hkv", [(0, 32, 8), (0, 8, 1), (0, 6, 3), (0, 4, 2), (0, 5, 5),
                                          (1, 2, 2)])
def test_device_plan_equals_host_plan_on_random_metadata(gpu_lib, dtype, hq, hkv):
    rng = np.random.default_rng(100 + 7 * hq + hkv + dtype)
    for trial in range(30):
        causal = trial % 6 != 5
        nseq = int(rng.integers(1, 13))
        nch = int(rng.integers(1, 9))
        lq = rng.integers(0, 700, size=nseq)
        # equal-cost ties on purpose in some trials: repeated lengths and offsets
        if trial % 3 == 0:
            lq[:] = lq[0]
        cu_q = wl.cu_from_lengths(lq)
        q_off = rng.integers(0, 2000, size=nseq).astype(np.int32)
        cu_ks = [wl.cu_from_lengths(rng.integers(0, 900, size=nseq)) for _ in range(nch)]
        k_offs = [rng.integers(0, 2500, size=nseq).astype(np.int32) for _ in range(nch)]
        host, devp = _host_and_device(gpu_lib, cu_q, cu_ks, q_off, k_offs, hq=hq, hkv=hkv,
                                      d=128 if dtype == 0 else 64, dtype=dtype, causal=causal)
        assert host.tobytes() == devp.tobytes(), (trial, nseq, nch, causal)


@pytest.mark.parametrize("name,seed", [("cp4_share", 0), ("cp4_share", 3), ("ctx128k_share", 0),
                                       ("pack", 0), ("pack", 4), ("tiny", 0)])
def test_device_plan_equals_host_plan_on_the_workloads(gpu_lib, name, seed):
    w = wl.make(name, seed)
    g = w.groups[0]
    host, devp = _host_and_device(gpu_lib, g.cu_q, [c.cu_k for c in g.chunks], g.q_off,
                                  [c.k_off for c in g.chunks], hq=w.hq, hkv=w.hkv, d=w.d,
                                  dtype=0 if w.dtype == "bf16" else 1)
    assert host.tobytes() == devp.tobytes()


def test_device_planner_refuses_metadata_beyond_its_argument(gpu_lib):
    cu = wl.cu_from_lengths([3] * 300)
    with pytest.raises(gpu_lib.CpattnError) as e:
        gpu_lib.cpattn_plan_build_device(cu, [cu], None, None, hq=4, hkv=2, d=64)
    assert e.value.status == 2


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", ["three", "one", "limit"])
def test_device_plan_equals_host_plan_up_to_its_tile_limit(gpu_lib, case, d):
    """Thousands of tiles (the sort runs over padded power-of-two key arrays), three chunks at
    staggered offsets so that totals tie in long runs; the last case has exactly the planner's
    limit of 4,096 tiles."""
    tt = _tile_tokens(gpu_lib, hq=32, hkv=8, d=d)
    lengths = {"three": [40000, 37000, 44000], "one": [131072], "limit": [4095 * tt - 8, 3]}[case]
    cu_q = wl.cu_from_lengths(lengths)
    nseq = len(lengths)
    q_off = np.full(nseq, 3 * 4096, np.int32)
    cu_ks = [wl.cu_from_lengths([4096 + 17 * c] * nseq) for c in range(3)]
    k_offs = [np.full(nseq, 4096 * c + 5 * c, np.int32) for c in range(3)]
    host, devp = _host_and_device(gpu_lib, cu_q, cu_ks, q_off, k_offs, hq=32, hkv=8, d=d)
    n_tiles = sum((n + tt - 1) // tt for n in lengths)
    assert len(host) == n_tiles * 3
    assert case != "limit" or n_tiles == 4096
    assert host.tobytes() == devp.tobytes()


@pytest.mark.parametrize("d", [128, 64])
def test_device_planner_refuses_plans_beyond_its_tile_limit(gpu_lib, d):
    tt = _tile_tokens(gpu_lib, hq=32, hkv=8, d=d)
    cu = wl.cu_from_lengths([4096 * tt + 1])      # 4097 tiles
    with pytest.raises(gpu_lib.CpattnError) as e:
        gpu_lib.cpattn_plan_build_device(cu, [cu], None, None, hq=32, hkv=8, d=d)
    assert e.value.status == 2


def test_device_planned_forward_captured_and_replayed(gpu_lib):
    """cpattn_fwd_chunks with device-planned metadata (the CP4 share of seed 2) captured into
    a graph: every replay, with eager work and synchronisation between replays and inputs
    changed in place between them, equals the eager call on the same inputs bit for bit."""
    import torch
    w = wl.make("cp4_share", 2)
    g = w.groups[0]
    q = dev(g.q, "bfloat16")
    ks = [dev(c.k, "bfloat16") for c in g.chunks]
    vs = [dev(c.v, "bfloat16") for c in g.chunks]
    meta = (g.cu_q, [c.cu_k for c in g.chunks], g.q_off, [c.k_off for c in g.chunks])
    tq, hq, d = q.shape
    nseq = len(g.cu_q) - 1
    ws = torch.zeros(gpu_lib.cpattn_workspace_size_chunks(nseq, g.cu_q, hq, w.hkv, d, len(ks)),
                     dtype=torch.uint8, device="cuda")
    o = torch.zeros((tq, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((hq, tq), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        graph.capture_begin()
        gpu_lib.cpattn_fwd_chunks(q, ks, vs, *meta, out=o, lse=lse, workspace=ws, stream=s)
        graph.capture_end()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(9)
    for rep in range(4):
        if rep:
            # new inputs in place (eager work between replays)
            q.copy_(torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_eager, l_eager = gpu_lib.cpattn_fwd_chunks(q, ks, vs, *meta)
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(lse, l_eager), rep
