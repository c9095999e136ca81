"""The fused forward inside a captured HIP graph (torch.cuda.CUDAGraph over
the HIP runtime).  The library allocates nothing, never synchronises and
enqueues no memset, so one forward captures as one graph of kernel nodes.
Every replay must equal the eager forward bit for bit (the kernels are
deterministic), with eager forwards, fills and synchronisations between the
replays."""

import pytest
import torch

import fp8_block_quantized_amd as moe
from synth import make_activations, make_weights
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,I,E,k", [
    (3, 512, 512, 64, 8),       # decode blocks, the second GEMM split over 4 K slices
    (32, 2048, 256, 128, 8),    # decode blocks, 136 x 8 weight tiles: no K slices
    (300, 384, 256, 2, 1),      # 128-row blocks: the persistent second GEMM
])
def test_graph_replay_matches_eager(T, H, I, E, k):
    note(f"graph capture T={T} H={H} I={I} E={E} k={k}")
    w13, w13s, w2, w2s = make_weights(H, I, E, 500 + T + E, "cuda")
    x, logits = make_activations(H, E, T, 7000 + T, "normal", "cuda")
    ws_e = moe.alloc_workspace(T, H, I, E, k)
    ws_g = moe.alloc_workspace(T, H, I, E, k)
    eager = moe.moe_fp8_forward(x, logits, w13, w13s, w2, w2s, k, True, workspace=ws_e).clone()
    torch.cuda.synchronize()

    out_g = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_fp8_forward(x, logits, w13, w13s, w2, w2s, k, True, out=out_g, workspace=ws_g)
    torch.cuda.synchronize()

    for rep in range(4):
        out_g.fill_(float("nan"))            # eager work between replays
        ws_g.fill_(0xA5)                     # every intermediate is rewritten by the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        again = moe.moe_fp8_forward(x, logits, w13, w13s, w2, w2s, k, True, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), eager.view(torch.int16)), f"eager after {rep}"


def test_graph_replay_batched_experts():
    """The batched (masked) expert format captured once and replayed with new
    device-side counts written between replays: each replay equals the eager
    call on the same counts (graph-capturable decode)."""
    E, M, H, I = 4, 32, 256, 256
    note(f"graph capture batched E={E} M={M} H={H} I={I}")
    w = make_weights(H, I, E, 901, "cuda")
    g = torch.Generator(device="cpu").manual_seed(902)
    x = torch.randn((E, M, H), generator=g).to(torch.bfloat16).cuda()
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    n = moe.moe_fp8_batched_workspace_bytes(E, M, H, I)
    ws_e = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(n, dtype=torch.uint8, device="cuda")
    out_g = torch.empty_like(x)
    counts.copy_(torch.tensor([5, 0, 32, 17], dtype=torch.int32))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_fp8_batched_experts(x, counts, *w, out=out_g, workspace=ws_g)
    torch.cuda.synchronize()
    for rep, cnt in enumerate([[5, 0, 32, 17], [32, 32, 1, 0], [0, 0, 0, 9], [7, 13, 21, 32]]):
        counts.copy_(torch.tensor(cnt, dtype=torch.int32))      # eager work between replays
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = moe.moe_fp8_batched_experts(x, counts, *w, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), eager.view(torch.int16)), f"replay {rep}, counts {cnt}"
