"""HIP-graph capture of the forward, for callers that replay a recorded launch sequence.

dcn_forward (with a caller workspace allocated before the capture) and
dcn_forward_noalloc (no workspace at all) are recorded once on torch's capture stream
and replayed several times.  Between replays the inputs are changed in place and other
eager work runs (a fill of the output, the reference call), with synchronisation; every
replay must equal an eager dcn_forward call on the same inputs bit for bit (the graph
holds the same kernels with the same arguments).  Cases: the box kernel with its
staging launch (c4), the direct kernel (tiny), and the bf16 and fp32 tile kernels."""

import pytest
import torch

import deformable_convolution_vision_amd as dcn
from deformable_convolution_vision_amd.workloads import WORKLOADS, custom, generate
from gpu_common import to_gpu

pytestmark = pytest.mark.gpu

CASES = {
    "c4": lambda: WORKLOADS["c4"],
    "tiny": lambda: WORKLOADS["tiny"],
    "tile_bf16": lambda: custom("graph_tile_bf16", "bf16", 2, 40, 19, 23, 32, 3, 1, 1, 1, 19, 23, seed=31),
    "tile_f32": lambda: custom("graph_tile_f32", "f32", 1, 24, 9, 10, 33, 3, 2, 1, 1, 5, 5, seed=32),
}


def _eager(desc, g, shape):
    nb = dcn.dcn_workspace_bytes(desc)
    out = torch.empty(shape, dtype=g["x"].dtype, device="cuda")
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda") if nb else None
    dcn.dcn_forward(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out, ws, nb)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name, noalloc):
    w = CASES[name]()
    print(f"[gpu-test] graph {name} noalloc={noalloc}", flush=True)
    g = to_gpu(generate(w))
    desc = dcn.describe(g["x"], g["weight"], w.stride, w.pad, w.dilation, g["offset"])
    nb = dcn.dcn_workspace_bytes(desc)
    if noalloc and nb > dcn.NOALLOC_SCRATCH_BYTES:
        pytest.skip("workspace larger than the no-allocation scratch array")
    shape = (w.B, w.Cout, w.Ho, w.Wo)
    out = torch.empty(shape, dtype=g["x"].dtype, device="cuda")
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    x0, off0 = g["x"].clone(), g["offset"].clone()

    def call():
        if noalloc:
            dcn.dcn_forward_noalloc(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out)
        else:
            dcn.dcn_forward(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out,
                            ws if nb else None, nb)

    # one eager call on a side stream first (the no-allocation path looks up its scratch
    # array on its first call on a device, which is no stream operation to record)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for i, (sx, so) in enumerate([(1.0, 1.0), (-0.5, 0.5), (2.0, -1.25), (1.0, 1.0)]):
        g["x"].copy_((x0.float() * sx).to(x0.dtype))
        g["offset"].copy_((off0.float() * so).to(off0.dtype))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ref = _eager(desc, g, shape)
        assert torch.equal(out, ref), f"{name}: replay {i} differs from the eager call"
    del graph
