"""colibri_moe_forward_static (working memory in the library's fixed per-GPU
array, no allocation) against colibri_moe_forward (working memory in the
handle) through the C ABI: both run the same kernels with the same launch
decisions, so y and every routing output must be bit-identical. Two calls in a
row on each handle, the second with a smaller batch (the array keeps the first
call's contents), then the ordinary entry point again on the same inputs; and a
batch whose working memory exceeds the array is refused before anything runs.
"""
import numpy as np
import pytest

import synth
from moe_case import compare, make_layer, run_gpu, to_dev

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
CASES = [
    (C("tiled-bf16", 600, 256, 8, 2, 512, "bf16", {1: 0.5}), 0),
    (C("small-batch-bf16", 40, 512, 8, 2, 1024, "bf16"), 0),
    (C("fine-grained-like", 700, 256, 64, 4, 256, "bf16"), 0),
    (C("fp32", 77, 256, 6, 3, 192, "f32", {2: 0.3}), 0),
    (C("fp8-weights", 300, 256, 8, 2, 512, "bf16"), 1 << 2),
]


def run_static(layer, x: np.ndarray) -> dict:
    import torch

    from moe_case import to_f64

    T = x.shape[0]
    rt = layer.routing_buffers(T)
    # only some routing outputs supplied: the rest live in the static array
    rt = {k: rt[k] for k in ("topk_ids", "topk_w", "perm", "expert_counts")}
    y = layer.forward(to_dev(x), routing=rt, static_scratch=True)
    torch.cuda.synchronize()
    out = {n: v.cpu().numpy() for n, v in rt.items()}
    out["y"] = to_f64(y)
    return out


@pytest.mark.parametrize("cfg,flags", CASES, ids=[c.name for c, _ in CASES])
def test_static_scratch_matches_forward(cfg, flags):
    print(f"static-scratch case {cfg} flags {flags}", flush=True)
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp, flags=flags)
    x = inp["x"]
    small = x[: cfg.T // 3 + 1]
    s1 = run_static(layer, x)
    s2 = run_static(layer, small)
    r1 = run_gpu(layer, x)
    r2 = run_gpu(layer, small)
    s3 = run_static(layer, x)
    layer.close()
    for s, r in ((s1, r1), (s2, r2), (s3, r1)):
        for key in s:
            assert np.array_equal(s[key], r[key]), key
    if flags == 0:
        print(compare(cfg, inp, r1), flush=True)


def test_static_scratch_refuses_batches_that_do_not_fit():
    import torch

    import sparse_moe_gemm_amd as cm

    # bf16, k = 2, d = 1024, d_ff = 4096: about 32 KiB of working memory per
    # token, so 2200 tokens need more than the 64 MiB array
    cfg = C("too-large", 2200, 1024, 4, 2, 4096, "bf16")
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = to_dev(inp["x"])
    y = torch.full_like(x, 7.0)
    st = cm.colibri_moe_forward_static(layer.handle, x.data_ptr(), cfg.T, y.data_ptr())
    assert st == cm.ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0)), "a refused call wrote y"
    # a batch that fits still runs and matches forward
    T = 256
    ys = torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda")
    yr = torch.empty_like(ys)
    assert cm.colibri_moe_forward_static(layer.handle, x.data_ptr(), T, ys.data_ptr()) == cm.OK
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), T, yr.data_ptr()) == cm.OK
    torch.cuda.synchronize()
    layer.close()
    assert torch.equal(ys, yr)
