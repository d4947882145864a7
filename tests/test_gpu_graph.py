"""The backward calls captured in a HIP graph: every workload's prepared call
(dense D=64 and D=128, packed, selected) is captured once and replayed
several times, with the program's own device work and synchronisations
between the replays; every replay must give the eager result bit for bit
(the default dQ mode and the selected path are deterministic).  The calls
launch kernels only (no memset, no allocation, no host synchronisation), so
the workspace-resident index, offsets and row statistics are rebuilt by the
replayed kernels themselves."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_graph_replays_match_eager(cid):
    wl, prep, _host = bench.build_inputs(cid)
    call, outs = prep(0)
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    # a prepared call launches on the stream current when it was prepared
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        gcall, outs = prep(0)
        gcall()                              # warm-up on the capturing stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            gcall()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for replay in range(3):
        for t in outs:                       # eager device work between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("dq", "dk", "dv"), outs, eager):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
                f"{wl.name} replay {replay}: {name} differs from the eager call"
