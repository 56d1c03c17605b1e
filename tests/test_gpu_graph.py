"""w4a16_gemm captured into a HIP graph: the header says calls may be
captured (no allocation, no synchronization, no host copies, counters reset
inside the kernels).  Each replay is checked bit for bit against the eager
result, with eager calls that share the workspace run between the replays."""
import pytest
import torch

import w4a16_synth as synth

from gpu_helpers import OnDevice, env, lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (variant, M, K, N): split-K with column blocks shared between workgroups,
# split-K with whole blocks, the tiled kernel with split K
CASES = [("splitk", 1, 4096, 4096), ("splitk", 8, 8192, 8192), ("splitk", 3, 1024, 28672),
         ("tiled", 70, 4096, 1024)]


def test_graph_replays_match_eager():
    w4 = lib()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    runs = []
    for i, (var, M, K, N) in enumerate(CASES):
        p = synth.make_problem(M, K, N, G=128, dtype="fp16", sym=False, seed=100 + i)
        with env(W4A16_FORCE_VARIANT=var):
            assert w4.w4a16_workspace_bytes(M, N, K, 128, 0) <= ws.numel()
            d = OnDevice(p)
            Y_eager = w4.w4a16_gemm(d.X, d.packed, workspace=ws)
            torch.cuda.synchronize()
        runs.append((var, d, Y_eager.clone(), torch.empty_like(Y_eager)))
    say("capturing the graph")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for var, d, _, Y in runs:
            with env(W4A16_FORCE_VARIANT=var):
                w4.w4a16_gemm(d.X, d.packed, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for var, d, _, Y in runs:
            Y.fill_(0)
        say(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for var, d, Y_eager, Y in runs:
            assert torch.equal(Y.view(torch.int16), Y_eager.view(torch.int16)), (rep, var)
        # eager calls on the same workspace between replays
        for var, d, Y_eager, _ in runs:
            with env(W4A16_FORCE_VARIANT=var):
                Y2 = w4.w4a16_gemm(d.X, d.packed, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(Y2.view(torch.int16), Y_eager.view(torch.int16)), (rep, var, "eager")
        assert int(ws[:65536].count_nonzero()) == 0, "counters not reset"
