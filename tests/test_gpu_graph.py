"""The forward captured into a HIP graph (torch.cuda.graph on the stream the
handle was created with) and replayed: every replay must give the eager
forward's outputs bit for bit, with eager forwards of other inputs and
synchronizations between the replays. Both GEMM paths (small-batch and tiled,
also enqueued together with the choice made on the device) and the
static-scratch entry point's kernels are covered; the forward enqueues
kernels only (no memset, no allocation, no synchronization in ASYNC mode)."""
import numpy as np
import pytest

import synth
from moe_case import to_dev

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
CASES = [
    C("decode-small", 32, 512, 8, 2, 1024, "bf16"),
    C("mixtral-small", 700, 256, 8, 2, 512, "bf16", {1: 0.5}),
    C("fine-grained-small", 1000, 256, 128, 4, 256, "bf16"),
    # both GEMM paths enqueued, the device picks the small-batch kernels
    C("both-paths-small", 200, 256, 64, 2, 256, "bf16"),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(cfg):
    import torch

    import sparse_moe_gemm_amd as cm

    print(f"graph case {cfg}", flush=True)
    inp = synth.make_inputs(cfg)
    s = torch.cuda.Stream()
    layer = cm.MoELayer(to_dev(inp["w_router"]), to_dev(inp["b_router"]), to_dev(inp["w_gate"]),
                        to_dev(inp["w_up"]), to_dev(inp["w_down"]), cfg.k, max_tokens=cfg.T,
                        flags=cm.FLAG_ASYNC, stream=s)
    x = to_dev(inp["x"])
    x2 = torch.flip(x, dims=[0]).contiguous()
    y = torch.empty_like(x)
    ids = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(s):
        layer.forward(x, y, {"topk_ids": ids})
    torch.cuda.synchronize()
    y_eager, ids_eager = y.clone(), ids.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        layer.forward(x, y, {"topk_ids": ids})
    torch.cuda.synchronize()
    y_other = torch.empty_like(x)
    for r in range(4):
        y.zero_()
        ids.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(ids, ids_eager), f"replay {r}"
        with torch.cuda.stream(s):  # eager work on other inputs between replays
            layer.forward(x2, y_other)
        torch.cuda.synchronize()
    del graph
    layer.close()
    assert not torch.equal(y_other, y_eager)
