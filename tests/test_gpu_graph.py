"""w4a16_gemm captured into a HIP graph: the header says calls may be
captured (no allocation, no synchronization, no host copies, counters reset
inside the kernels).  Each replay is checked bit for bit against the eager
result, with eager calls that share the workspace run between the replays."""
import pytest
import torch

import w4a16_synth as synth

from gpu_helpers import OnDevice, lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (plan, M, K, N): the decode kernel (several items per workgroup), the wide
# kernel (whole blocks, and K split into parts across workgroups), split-K
# with column blocks shared between workgroups, split-K with whole blocks, the
# tiled kernel with split K
CASES = [("decode", 1, 8192, 28672), (("decode", 3), 4, 2048, 1024),
         ("wide", 64, 4096, 1024), (("wide", 255), 100, 2048, 512),
         ("splitk", 1, 4096, 4096), ("splitk", 8, 8192, 8192), ("splitk", 3, 1024, 28672),
         ("tiled", 70, 4096, 1024)]


def test_graph_replays_match_eager():
    w4 = lib()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    runs = []
    for i, (var, M, K, N) in enumerate(CASES):
        p = synth.make_problem(M, K, N, G=128, dtype="fp16", sym=False, seed=100 + i)
        assert w4.w4a16_workspace_bytes(M, N, K, 128, w4.plan_flags(var)) <= ws.numel()
        d = OnDevice(p)
        Y_eager = w4.w4a16_gemm(d.X, d.packed, workspace=ws, plan=var)
        torch.cuda.synchronize()
        runs.append((var, d, Y_eager.clone(), torch.empty_like(Y_eager)))
    say("capturing the graph")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for var, d, _, Y in runs:
            w4.w4a16_gemm(d.X, d.packed, Y=Y, workspace=ws, plan=var)
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
            Y2 = w4.w4a16_gemm(d.X, d.packed, workspace=ws, plan=var)
            torch.cuda.synchronize()
            assert torch.equal(Y2.view(torch.int16), Y_eager.view(torch.int16)), (rep, var, "eager")
        assert int(ws[:65536].count_nonzero()) == 0, "counters not reset"


def test_fused_ffn_block_graph_matches_eager():
    """A decoder FFN block, G = silu(X Wg), H = (X Wu) * G, Y = H Wd + X, as
    three epilogue-fused calls captured in one graph: every replay equals the
    eager chain bit for bit."""
    w4 = lib()
    M, Hd, F, G = 4, 1024, 2048, 128
    flags = w4.flags_of("fp16", False)
    dev = torch.device("cuda")
    blobs = []
    for seed, (K, N) in ((21, (Hd, F)), (22, (Hd, F)), (23, (F, Hd))):
        p = synth.make_problem(1, K, N, G=G, dtype="fp16", sym=False, seed=seed)
        _, qw, sc, zr = w4.to_device(p, dev)
        blobs.append(w4.w4a16_repack(qw, sc, zr, K, N, G, flags))
    X = torch.from_numpy(synth.make_activations(M, Hd, "fp16", seed=5).view("int16")).view(
        torch.float16).to(dev)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    Gt = torch.empty((M, F), dtype=torch.float16, device=dev)
    Ht = torch.empty_like(Gt)
    Y = torch.empty((M, Hd), dtype=torch.float16, device=dev)

    def block():
        w4.w4a16_gemm_ex(X, blobs[0], Y=Gt, workspace=ws, activation="silu")
        w4.w4a16_gemm_ex(X, blobs[1], Y=Ht, workspace=ws, aux=Gt, aux_op="mul")
        w4.w4a16_gemm_ex(Ht, blobs[2], Y=Y, workspace=ws, aux=X, aux_op="add")

    block()
    torch.cuda.synchronize()
    Y_eager = Y.clone()
    assert torch.isfinite(Y_eager.float()).all()
    say("capturing the FFN block")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block()
    torch.cuda.synchronize()
    for rep in range(3):
        Y.fill_(0)
        Gt.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_eager.view(torch.int16)), rep
        block()   # eager between replays, on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_eager.view(torch.int16)), (rep, "eager")
