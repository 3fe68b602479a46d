"""The library's per-stream workspaces on the GPU: kept between calls,
grown when a call needs more, separate per stream, freed on request, and
replaced by stream-ordered allocations under graph capture.

Each case compares whole outputs bit for bit with fhd_compute_noalloc,
whose temporaries live in the library's static scratch array instead (the
same kernels and split counts, so the same bits), and samples the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, inputs, metrics

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def on_device(case):
    return [torch.from_numpy(np.ascontiguousarray(case[k])).to(DEV)
            for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")]


def reference(t):
    """F^H D through the no-allocation entry point (static scratch)."""
    N = t[5].numel()
    rr, ri = torch.empty(N, device=DEV), torch.empty(N, device=DEV)
    binding.fhd_compute_noalloc(*t, rr, ri)
    torch.cuda.synchronize(DEV)
    return rr, ri


def check_oracle(case, got, name):
    idx = inputs.voxel_subset(case["x"].size, min(512, case["x"].size), seed=951)
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"],
                     case["x"][idx], case["y"][idx], case["z"][idx])
    e = metrics.rel_l2(got[0].cpu().numpy()[idx], got[1].cpu().numpy()[idx], *ref)
    assert e <= 5e-4, (name, e)


CASES = [("spiral32", lambda: inputs.make_workload("spiral32")),
         ("random 5000 x 123", lambda: inputs.random_case(5000, 123, seed=952)),
         ("random16", lambda: inputs.make_workload("random16")),
         ("radial64", lambda: inputs.make_workload("radial64"))]


def test_kept_workspace_across_calls_of_changing_size():
    """Small, larger, smaller, largest, then the first again, on one
    stream: every call matches the scratch-array path bit for bit."""
    order = [0, 1, 2, 3, 0]
    made = {}
    for i in order:
        name, make = CASES[i]
        if name not in made:
            made[name] = make()
        c = made[name]
        t = on_device(c)
        print("kept workspace: %s" % name, flush=True)
        got = binding.fhd_compute(*t)
        torch.cuda.synchronize(DEV)
        want = reference(t)
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), name
        check_oracle(c, got, name)


def test_two_streams_keep_separate_workspaces():
    """Two streams, each with its own inputs, their calls enqueued in turn
    with no synchronisation between them."""
    ca, cb = inputs.make_workload("spiral32"), inputs.random_case(6000, 777, seed=953)
    ta, tb = on_device(ca), on_device(cb)
    want_a, want_b = reference(ta), reference(tb)
    sa, sb = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    outs = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            ra = binding.fhd_compute(*ta)
        with torch.cuda.stream(sb):
            rb = binding.fhd_compute(*tb)
        outs.append((ra, rb))
    torch.cuda.synchronize(DEV)
    for ra, rb in outs:
        assert torch.equal(ra[0], want_a[0]) and torch.equal(ra[1], want_a[1])
        assert torch.equal(rb[0], want_b[0]) and torch.equal(rb[1], want_b[1])


def test_release_then_call_again():
    c = inputs.make_workload("spiral32")
    t = on_device(c)
    first = binding.fhd_compute(*t)
    torch.cuda.synchronize(DEV)
    binding.fhd_release_workspaces()
    again = binding.fhd_compute(*t)
    torch.cuda.synchronize(DEV)
    assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])


@pytest.mark.parametrize("name", ["spiral32", "random 5000 x 123"])
def test_graph_capture_replays_match_eager(name):
    """fhd_compute captured into a graph (its temporaries become the
    graph's own allocations), replayed three times with eager work and
    synchronisation between the replays: every replay matches the eager
    result bit for bit."""
    c = dict(CASES)[name]()
    t = on_device(c)
    N = t[5].numel()
    eager = reference(t)
    rr, ri = torch.empty(N, device=DEV), torch.empty(N, device=DEV)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        binding.fhd_compute(*t, rr, ri)   # warm-up outside the capture
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        binding.fhd_compute(*t, rr, ri)
    torch.cuda.synchronize(DEV)
    for k in range(3):
        rr.fill_(float("nan"))
        ri.fill_(float("nan"))
        binding.fhd_compute(*t)   # eager work on the same device in between
        torch.cuda.synchronize(DEV)
        print("graph replay %d of %s" % (k, name), flush=True)
        g.replay()
        torch.cuda.synchronize(DEV)
        assert torch.equal(rr, eager[0]) and torch.equal(ri, eager[1]), (name, k)
