"""Calls that enqueue both GEMM paths: more tokens than the small-batch row
limit (CMOE_DECODE_MAX_ROWS, default 48 rows, 32 with 8-bit weights) and at
most CMOE_DECODE_MAX_A assignments. The kernels read the expert offsets and
the small-batch ones take the call when no expert holds more rows than the
limit, the tiled ones otherwise; the combine reads the chosen path's expert
outputs. So y and every routing output must equal, bit for bit, those of the
chosen path forced alone, and (bf16 weights) pass the oracle comparison.
Cases are built so that each choice occurs: many experts with few rows each
(small-batch), and hot experts (tiled)."""
import numpy as np
import pytest

import synth
from moe_case import compare, make_layer, run_gpu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
FORCED = {"tiled": {"CMOE_DECODE_MAX_A": "0"},
          "small-batch": {"CMOE_DECODE_MAX_A": "65536", "CMOE_DECODE_MAX_ROWS": "0"}}
WEIGHTS = {"bf16": 0, "fp8-weights": 1 << 2, "w8a8": (1 << 2) | (1 << 3)}
# (layer, the path the device must choose)
CASES = [
    (C("many-experts", 200, 256, 64, 2, 256, "bf16"), "small-batch"),
    (C("e8-moderate", 120, 256, 8, 2, 512, "bf16"), "small-batch"),
    (C("hot-experts", 160, 256, 16, 2, 256, "bf16", {0: 4.0, 3: 4.0}), "tiled"),
    (C("e8-large", 600, 256, 8, 2, 512, "bf16"), "tiled"),
    (C("k4-E128", 400, 256, 128, 4, 256, "bf16"), "small-batch"),
]


def _run(cfg, inp, flags, env, monkeypatch):
    with monkeypatch.context() as m:
        for key, val in env.items():
            m.setenv(key, val)
        layer = make_layer(cfg, inp, flags=flags)
    g = run_gpu(layer, inp["x"])
    layer.close()
    return g


@pytest.mark.parametrize("weights", list(WEIGHTS))
@pytest.mark.parametrize("cfg,want", CASES, ids=[c.name for c, _ in CASES])
def test_device_path_choice(cfg, want, weights, monkeypatch):
    print(f"dual-path case {cfg} weights {weights}", flush=True)
    monkeypatch.delenv("CMOE_DECODE_MAX_A", raising=False)
    monkeypatch.delenv("CMOE_DECODE_MAX_ROWS", raising=False)
    flags = WEIGHTS[weights]
    limit = 48 if flags == 0 else 32
    assert cfg.T > limit and cfg.T * cfg.k <= 2048, "both paths enqueued by default"
    inp = synth.make_inputs(cfg)
    g = _run(cfg, inp, flags, {}, monkeypatch)
    most = int(g["expert_counts"].max())
    chosen = "small-batch" if most <= limit else "tiled"
    # the case is what it claims (with 8-bit weights the limit is lower)
    if flags == 0:
        assert chosen == want, f"most rows {most}"
    ref = _run(cfg, inp, flags, FORCED[chosen], monkeypatch)
    for key in g:
        assert np.array_equal(g[key], ref[key]), f"{key} differs from the {chosen} path alone (most rows {most})"
    if flags == 0:
        print(chosen, most, compare(cfg, inp, g), flush=True)
    else:
        print(chosen, most, flush=True)


def test_row_limit_boundary(monkeypatch):
    """The device compares the largest expert's rows with the limit
    inclusively: a limit equal to that count takes the small-batch path, one
    less the tiled path (both with every call enqueueing both paths)."""
    cfg = C("e8-moderate", 120, 256, 8, 2, 512, "bf16")
    print(f"dual-path boundary case {cfg}", flush=True)
    monkeypatch.delenv("CMOE_DECODE_MAX_A", raising=False)
    inp = synth.make_inputs(cfg)
    small = _run(cfg, inp, 0, FORCED["small-batch"], monkeypatch)
    tiled = _run(cfg, inp, 0, FORCED["tiled"], monkeypatch)
    most = int(tiled["expert_counts"].max())
    assert 1 < most < cfg.T and not np.array_equal(small["y"], tiled["y"])
    for limit, ref in ((most, small), (most - 1, tiled)):
        g = _run(cfg, inp, 0, {"CMOE_DECODE_MAX_ROWS": str(limit)}, monkeypatch)
        for key in g:
            assert np.array_equal(g[key], ref[key]), f"limit {limit}, most rows {most}: {key}"


def test_fused_combine_handle_alternating_calls(monkeypatch):
    """A handle with the combine fused into the tiled down GEMM
    (CMOE_FUSE_COMBINE=1): calls that enqueue both paths run the combine as
    its own kernel, tiled-only calls (more than CMOE_DECODE_MAX_A assignments)
    fuse it. Alternating the two must match a handle without the fusion bit
    for bit, so the fused combine's arrival counts stay at zero between
    calls."""
    cfg = C("alternating", 1200, 256, 8, 2, 512, "bf16")
    print(f"dual-path fused-combine case {cfg}", flush=True)
    monkeypatch.delenv("CMOE_DECODE_MAX_A", raising=False)
    monkeypatch.delenv("CMOE_DECODE_MAX_ROWS", raising=False)
    inp = synth.make_inputs(cfg)
    x = inp["x"]
    sizes = [300, cfg.T, 60, cfg.T, 300]  # 600 and 120 assignments: both paths; 2400: tiled only
    outs = {}
    for fuse in ("0", "1"):
        monkeypatch.setenv("CMOE_FUSE_COMBINE", fuse)
        layer = make_layer(cfg, inp)
        outs[fuse] = [run_gpu(layer, x[:n]) for n in sizes]
        layer.close()
    for i, (a, b) in enumerate(zip(outs["0"], outs["1"])):
        for key in a:
            assert np.array_equal(a[key], b[key]), f"call {i} ({sizes[i]} tokens): {key}"
    print(compare(cfg, inp, outs["1"][1]), flush=True)
