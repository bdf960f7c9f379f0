"""GPU parity of the whole layer through the C ABI against the CPU oracle.

Small cases (every token checked) keep the shapes of the five workloads at
sizes the oracle finishes in seconds, with several m- and n-tiles per expert and
ragged tails; the full-size workloads (the five layer shapes and the masked
skewed variant, in the launch configuration the benchmark times) check routing,
dispatch and the output on every token.
"""
import numpy as np
import pytest

import synth
from moe_case import compare, make_layer, run_gpu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
SMALL = [
    synth.CONFIGS["tiny-f32"],
    C("mixtral-small", 700, 256, 8, 2, 512, "bf16"),
    C("fine-grained-small", 1000, 256, 128, 4, 256, "bf16"),
    C("decode-small", 32, 512, 8, 2, 1024, "bf16"),
    C("skewed-small", 2000, 256, 64, 2, 128, "bf16", {0: 4.0, 3: 4.0}),
    C("skewed-masked-small", 2000, 256, 64, 2, 128, "bf16",
      {0: 4.0, 3: 4.0, **{e: -1.0e4 for e in range(44, 64)}}),
    C("f32-ragged", 77, 256, 6, 3, 192, "f32", {2: 0.3}),
    C("one-token", 1, 128, 8, 2, 128, "bf16"),
    C("ragged-17", 17, 384, 16, 3, 384, "bf16"),
    C("single-expert", 130, 128, 1, 1, 128, "bf16"),
    C("k-equals-E", 90, 256, 4, 4, 128, "bf16"),
    C("all-to-one", 300, 128, 8, 1, 128, "bf16", {5: 100.0}),
    C("k8-E256", 64, 128, 256, 8, 128, "bf16"),
    # more gate/up tiles than compute units (each workgroup walks several) and
    # an expert whose last m-tile has 6 rows: waves whose rows are all padding
    C("last-tile-padding", 1030, 256, 1, 1, 6656, "bf16"),
    # at least 4096 assignments: each expert's compaction is split over
    # several workgroups; one hot expert takes every token, the other none
    C("hot-expert-split-dispatch", 4608, 128, 2, 1, 128, "bf16", {0: 100.0}),
    C("split-dispatch-k4", 1100, 128, 16, 4, 128, "bf16", {3: 2.0}),
    # one expert with a ragged last m-tile of 1, 16, 17, 32 and 33 rows past
    # 256 (the last m-tile's waves: only the first holding rows, the first
    # two, all); 800 = 3 * 256 + 32 puts the ragged tile after full ones;
    # d = 384 runs the down GEMM's 128-column tiles
    C("tail-257", 257, 256, 1, 1, 512, "bf16"),
    C("tail-272", 272, 256, 1, 1, 512, "bf16"),
    C("tail-273", 273, 256, 1, 1, 512, "bf16"),
    C("tail-288", 288, 256, 1, 1, 512, "bf16"),
    C("tail-289", 289, 256, 1, 1, 512, "bf16"),
    C("tail-800", 800, 256, 1, 1, 768, "bf16"),
    C("tail-d384", 270, 384, 1, 1, 256, "bf16"),
    C("tails-mixed", 1100, 256, 4, 2, 256, "bf16", {0: 0.3, 1: -0.2}),
    # small experts (at most 64 rows) among big ones: the down GEMM spreads
    # their tiles over the big experts' tiles in units of 8 (a remainder of
    # each class at the end); two K splits (K = 2048) and one
    C("small-among-big", 3000, 256, 32, 2, 2048, "bf16", {0: 3.0, 5: 3.0, 9: 2.0}),
    C("small-among-big-k1", 2600, 256, 48, 1, 256, "bf16", {2: 4.0, 40: 4.0}),
    # at least 4096 tokens with 64 or 128 experts: router blocks of 64 or 32
    # tokens, the last one ragged (4 tokens, 1 token: its other rows are
    # clamped repeats whose results are dropped)
    C("router-64-token-blocks-ragged", 4100, 256, 64, 2, 128, "bf16", {7: 0.5}),
    C("router-32-token-blocks-ragged", 4097, 256, 128, 4, 128, "bf16"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_layer_parity(cfg):
    print(f"case {cfg}", flush=True)
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    g = run_gpu(layer, inp["x"])
    layer.close()
    rep = compare(cfg, inp, g)
    print(rep, flush=True)
    if cfg.name == "all-to-one":
        assert g["expert_counts"][5] == cfg.T and rep["empty_experts"] == cfg.E - 1
    if cfg.name == "skewed-masked-small":
        assert np.all(g["expert_counts"][44:] == 0)
    if cfg.name == "hot-expert-split-dispatch":
        assert g["expert_counts"][0] == cfg.T and g["expert_counts"][1] == 0


# Both bf16 GEMM paths on the same inputs: the tiled grouped GEMMs and the
# small-batch (weight streaming) path, forced through the init-time threshold
# CMOE_DECODE_MAX_A. The small-batch path is taken here also for batches far
# larger than it is meant for (several 32-token groups per expert, hot
# experts), which exercises its row-group loop and its K slices; one expert
# with 33, 65 and 130 rows puts a group pair or a lone group of 1 or 2 rows
# at the end.
# the small-batch path forced: every call within CMOE_DECODE_MAX_A, and no
# per-expert row test on the device (CMOE_DECODE_MAX_ROWS=0)
PATHS = {"tiled": {"CMOE_DECODE_MAX_A": "0"},
         "small-batch": {"CMOE_DECODE_MAX_A": "65536", "CMOE_DECODE_MAX_ROWS": "0"}}
BOTH = [
    C("decode-small", 32, 512, 8, 2, 1024, "bf16"),
    C("one-token", 1, 128, 8, 2, 128, "bf16"),
    C("ragged-17", 17, 384, 16, 3, 384, "bf16"),
    C("single-expert", 130, 128, 1, 1, 128, "bf16"),
    C("single-expert-33", 33, 128, 1, 1, 128, "bf16"),
    C("single-expert-65", 65, 128, 1, 1, 128, "bf16"),
    C("mixtral-small", 700, 256, 8, 2, 512, "bf16"),
    C("k8-E256", 64, 128, 256, 8, 128, "bf16"),
    C("skewed-small", 2000, 256, 64, 2, 128, "bf16", {0: 4.0, 3: 4.0}),
]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("cfg", BOTH, ids=[c.name for c in BOTH])
def test_both_gemm_paths(cfg, path, monkeypatch):
    for key, val in PATHS[path].items():
        monkeypatch.setenv(key, val)
    print(f"case {cfg} path {path}", flush=True)
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    g = run_gpu(layer, inp["x"])
    layer.close()
    print(compare(cfg, inp, g), flush=True)


# The combine fused into the down GEMM's epilogue (CMOE_FUSE_COMBINE=1, tiled
# bf16 path) against the combine kernel (the default): both add the
# same fp32 values in the same order, so y must be bit-identical, also with the
# K split of the down GEMM (mixtral-small), 128-column tiles (ragged-17, d=384)
# and k = 8; calls in a row and a smaller batch in between check that the
# arrival counts are back at zero after every call.
FUSED = [
    C("mixtral-small", 700, 256, 8, 2, 512, "bf16"),
    C("ragged-17", 17, 384, 16, 3, 384, "bf16"),
    C("k8-E256", 64, 128, 256, 8, 128, "bf16"),
    C("skewed-small", 2000, 256, 64, 2, 128, "bf16", {0: 4.0, 3: 4.0}),
    C("fine-grained-small", 1000, 256, 128, 4, 256, "bf16"),
]


WEIGHTS = {"bf16": 0, "fp8-weights": 1 << 2, "w8a8": (1 << 2) | (1 << 3)}


@pytest.mark.parametrize("weights", list(WEIGHTS))
@pytest.mark.parametrize("cfg", FUSED, ids=[c.name for c in FUSED])
def test_fused_combine_matches_combine_kernel(cfg, weights, monkeypatch):
    import sparse_moe_gemm_amd as cm

    assert WEIGHTS["w8a8"] == cm.FLAG_FP8_WEIGHTS | cm.FLAG_FP8_ACTIVATIONS
    if weights == "w8a8" and min(cfg.d, cfg.f) < 256:
        pytest.skip("8-bit activations need d_model, d_ff >= 256")
    monkeypatch.setenv("CMOE_DECODE_MAX_A", "0")
    print(f"case {cfg} {weights}", flush=True)
    inp = synth.make_inputs(cfg)
    monkeypatch.setenv("CMOE_FUSE_COMBINE", "0")
    plain = make_layer(cfg, inp, flags=WEIGHTS[weights])
    ref = run_gpu(plain, inp["x"])
    ref_small = run_gpu(plain, inp["x"][: cfg.T // 2 + 1])
    plain.close()
    monkeypatch.setenv("CMOE_FUSE_COMBINE", "1")
    fused = make_layer(cfg, inp, flags=WEIGHTS[weights])
    runs = [run_gpu(fused, inp["x"]), run_gpu(fused, inp["x"])]
    small = run_gpu(fused, inp["x"][: cfg.T // 2 + 1])
    runs.append(run_gpu(fused, inp["x"]))
    fused.close()
    for g in runs:
        for key in ref:
            assert np.array_equal(g[key], ref[key]), key
    for key in ref_small:
        assert np.array_equal(small[key], ref_small[key]), key
    if weights == "bf16":
        print(compare(cfg, inp, runs[0]), flush=True)


def test_empty_batch_and_errors():
    import torch

    import sparse_moe_gemm_amd as cm

    cfg = C("errs", 8, 128, 4, 2, 128, "bf16")
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp, max_tokens=8)
    x = torch.zeros(16, 128, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), 0, y.data_ptr()) == cm.OK
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), 9, y.data_ptr()) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), -1, y.data_ptr()) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr() + 2, 4, y.data_ptr()) == cm.ERR_ALIGNMENT
    assert cm.colibri_moe_forward(layer.handle, 0, 4, y.data_ptr()) == cm.ERR_INVALID_ARG
    # routing buffers: topk_ids must be 16-byte aligned, the others 4-byte
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    for field, off in (("topk_ids", 4), ("topk_ids", 8), ("perm", 2), ("logits", 1), ("topk_w", 2)):
        r = cm.Routing(**{field: buf.data_ptr() + off})
        assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), 4, y.data_ptr(), r) == cm.ERR_ALIGNMENT, field
    r = cm.Routing(topk_ids=buf.data_ptr() + 16, perm=buf.data_ptr() + 4)
    assert cm.colibri_moe_forward(layer.handle, x.data_ptr(), 4, y.data_ptr(), r) == cm.OK
    h = layer.handle
    layer.close()
    assert cm.colibri_moe_free(h) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward(h, x.data_ptr(), 4, y.data_ptr()) == cm.ERR_INVALID_ARG


def test_handle_reuse_with_smaller_batch_and_determinism():
    cfg = C("reuse", 500, 256, 16, 2, 256, "bf16", {1: 1.0})
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp, max_tokens=512)
    g1 = run_gpu(layer, inp["x"])
    g2 = run_gpu(layer, inp["x"][:123])
    g3 = run_gpu(layer, inp["x"])
    layer.close()
    for key in g1:
        assert np.array_equal(g1[key], g3[key]), f"{key} not bit-reproducible"
    fresh = make_layer(cfg, inp, max_tokens=123)
    g4 = run_gpu(fresh, inp["x"][:123])
    fresh.close()
    for key in g2:
        assert np.array_equal(g2[key], g4[key]), f"{key} depends on earlier calls"
    # Routing is per token, so it is the same in a smaller batch; the outputs
    # agree up to fp32 summation order (the GEMM path and its K split depend
    # on the batch size: here 500 tokens take the tiled GEMMs, 123 the
    # small-batch path).
    for key in ("topk_ids", "topk_w", "logits"):
        assert np.array_equal(g2[key], g1[key][:123]), key
    d = np.abs(g2["y"] - g1["y"][:123]).max()
    assert d <= 2e-2 * np.abs(g1["y"]).max(), d
    compare(cfg.with_(T=123), dict(inp, x=inp["x"][:123]), g2)


@pytest.mark.parametrize("E", [64, 128])
def test_routing_does_not_depend_on_batch_size(E):
    """The router takes 16, 32 or 64 tokens per block depending on the batch
    size and the expert count; a token's logits, experts and weights must not
    change with it (same bits), also for a token at another position in its
    block."""
    cfg = C(f"batch-invariance-E{E}", 4096, 512, E, 2, 128, "bf16")
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    print(f"routing batch invariance {cfg}", flush=True)
    full = run_gpu(layer, inp["x"])
    part = run_gpu(layer, inp["x"][37:137])
    layer.close()
    for key in ("logits", "topk_ids", "topk_w"):
        assert np.array_equal(part[key], full[key][37:137]), key


def test_partial_routing_outputs():
    import torch

    cfg = C("partial", 200, 256, 8, 2, 128, "bf16")
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    full = run_gpu(layer, inp["x"])
    from moe_case import to_dev, to_f64

    x = to_dev(inp["x"])
    y0 = to_f64(layer.forward(x))
    rt = layer.routing_buffers(cfg.T)
    some = {"perm": rt["perm"], "topk_w": rt["topk_w"]}
    y1 = to_f64(layer.forward(x, routing=some))
    torch.cuda.synchronize()
    layer.close()
    assert np.array_equal(y0, full["y"]) and np.array_equal(y1, full["y"])
    assert np.array_equal(some["perm"].cpu().numpy(), full["perm"])


FULL = ["tiny-f32", "mixtral", "fine-grained", "decode", "skewed", "skewed-masked"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    cfg = synth.CONFIGS[name]
    print(f"full-size case {cfg}", flush=True)
    inp = synth.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    g = run_gpu(layer, inp["x"])
    layer.close()
    rep = compare(cfg, inp, g)
    assert rep["tokens_checked"] == cfg.T
    print(name, rep, flush=True)
    if name == "decode":
        assert np.all(g["expert_counts"] > 0), "every expert is hit in the decode batch"
    if name == "skewed-masked":
        assert rep["empty_experts"] == 20


BY_NAME = {c.name: c for c in SMALL}
PLACEMENT = [BY_NAME[n] for n in ("mixtral-small", "fine-grained-small", "skewed-masked-small", "small-among-big")]


@pytest.mark.parametrize("cfg", PLACEMENT, ids=[c.name for c in PLACEMENT])
def test_xcd_contiguous_placement(cfg, monkeypatch):
    """CMOE_XCD_MAP=3 (read at init) gives each XCD one contiguous eighth of
    both GEMMs' tile orders. Placement changes which workgroup runs a tile,
    not how a tile sums, so every output is bit-identical to the default
    placement's, and both match the oracle."""
    inp = synth.make_inputs(cfg)
    print(f"xcd placement {cfg}", flush=True)
    plain = make_layer(cfg, inp)
    g0 = run_gpu(plain, inp["x"])
    plain.close()
    monkeypatch.setenv("CMOE_XCD_MAP", "3")
    placed = make_layer(cfg, inp)
    g1 = run_gpu(placed, inp["x"])
    placed.close()
    for key in g0:
        assert np.array_equal(g0[key], g1[key]), key
    compare(cfg, inp, g1)


STAGES64 = [BY_NAME[n] for n in ("mixtral-small", "fine-grained-small", "skewed-masked-small", "last-tile-padding",
                                  "tail-288", "small-among-big")]


@pytest.mark.parametrize("cfg", STAGES64, ids=[c.name for c in STAGES64])
def test_k64_stages_bit_identical(cfg, monkeypatch):
    """The 64-wide K stage kernel (CMOE_K64 bit 0: gate/up, the default for
    layers of at least 768 rows per expert; bit 1: down; bit 2: gate/up at
    any rows per expert) and the 32-wide one add the same products in the
    same order, so every output is bit-identical between CMOE_K64 = 0, 5 and
    7; all match the oracle."""
    inp = synth.make_inputs(cfg)
    print(f"k64 stages {cfg}", flush=True)
    outs = []
    for v in ("0", "5", "7"):
        monkeypatch.setenv("CMOE_K64", v)
        layer = make_layer(cfg, inp)
        outs.append(run_gpu(layer, inp["x"]))
        layer.close()
    for g in outs[1:]:
        for key in outs[0]:
            assert np.array_equal(outs[0][key], g[key]), key
    compare(cfg, inp, outs[1])
