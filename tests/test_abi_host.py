"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/colibri_moe.h declares, and rejects bad arguments before
it touches the device."""
import ctypes
import os
import re

import pytest

import sparse_moe_gemm_amd as cm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(colibri_moe_\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = cm.lib()
    names = declared_functions()
    assert len(names) >= 6
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(cm.EXPORTS)


def test_status_strings_and_stage_names():
    assert cm.colibri_moe_status_string(cm.OK) == "ok"
    texts = {cm.colibri_moe_status_string(s) for s in range(7)}
    assert len(texts) == 7
    assert cm.colibri_moe_status_string(99) == "unknown status"
    assert [cm.colibri_moe_stage_name(i) for i in range(6)] == list(cm.STAGES)
    assert cm.colibri_moe_stage_name(6) is None


def _cfg(**kw):
    base = dict(d_model=256, d_ff=128, n_experts=8, top_k=2, max_tokens=64, dtype=cm.BF16, flags=0)
    base.update(kw)
    return cm.Config(**base)


FAKE = 0x100000  # never dereferenced: validation fails before any use


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), cm.ERR_INVALID_ARG),
    (dict(top_k=9, n_experts=8), cm.ERR_INVALID_ARG),
    (dict(dtype=7), cm.ERR_INVALID_ARG),
    (dict(max_tokens=0), cm.ERR_INVALID_ARG),
    (dict(d_model=-128), cm.ERR_INVALID_ARG),
    (dict(n_experts=300, top_k=2), cm.ERR_UNSUPPORTED),
    (dict(n_experts=16, top_k=9), cm.ERR_UNSUPPORTED),
    (dict(d_model=192), cm.ERR_UNSUPPORTED),
    (dict(d_ff=100), cm.ERR_UNSUPPORTED),
    (dict(d_ff=192), cm.ERR_UNSUPPORTED),
    (dict(max_tokens=(1 << 24) + 1), cm.ERR_UNSUPPORTED),
    (dict(dtype=cm.F32, flags=cm.FLAG_FP8_WEIGHTS), cm.ERR_UNSUPPORTED),
    (dict(flags=cm.FLAG_FP8_ACTIVATIONS), cm.ERR_UNSUPPORTED),
    (dict(flags=cm.FLAG_FP8_WEIGHTS | cm.FLAG_FP8_ACTIVATIONS), cm.ERR_UNSUPPORTED),  # d_ff = 128
    (dict(d_model=128, d_ff=256, flags=cm.FLAG_FP8_WEIGHTS | cm.FLAG_FP8_ACTIVATIONS), cm.ERR_UNSUPPORTED),
])
def test_init_rejects_bad_configs(kw, status):
    w = cm.Weights(FAKE, None, FAKE, FAKE, FAKE)
    st, h = cm.colibri_moe_init(_cfg(**kw), w)
    assert st == status and not h


def test_init_rejects_null_and_misaligned_weights():
    st, _ = cm.colibri_moe_init(_cfg(), cm.Weights(FAKE, None, None, FAKE, FAKE))
    assert st == cm.ERR_INVALID_ARG
    st, _ = cm.colibri_moe_init(_cfg(), cm.Weights(FAKE + 8, None, FAKE, FAKE, FAKE))
    assert st == cm.ERR_ALIGNMENT
    L = cm.lib()
    assert L.colibri_moe_init(None, None, None, None) == cm.ERR_INVALID_ARG


def test_forward_and_free_reject_unknown_handles():
    assert cm.colibri_moe_free(None) == cm.OK
    assert cm.colibri_moe_free(FAKE) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward(None, FAKE, 4, FAKE) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward(FAKE, FAKE, 4, FAKE) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward_static(None, FAKE, 4, FAKE) == cm.ERR_INVALID_ARG
    assert cm.colibri_moe_forward_static(FAKE, FAKE, 4, FAKE) == cm.ERR_INVALID_ARG
    with pytest.raises(RuntimeError):
        cm.colibri_moe_stage_times(FAKE)


def test_static_scratch_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "colibri_moe.h")).read()
    m = re.search(r"#define COLIBRI_MOE_STATIC_SCRATCH_BYTES \((\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == cm.STATIC_SCRATCH_BYTES


def test_binding_is_marshalling_only():
    # The product package never imports the oracle or the input generator.
    pkg = os.path.join(ROOT, "sparse_moe_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower().replace("oracle-free", ""), fn
                assert "import synth" not in text and "moe_oracle" not in text, fn


@pytest.mark.parametrize("args,status", [
    ((None, 4, 8, FAKE, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE, 4, 8, None, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE, 4, 8, FAKE, None), cm.ERR_INVALID_ARG),
    ((FAKE, 0, 8, FAKE, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE, 4, 4, FAKE, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE, 4, 12, FAKE, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE, 1 << 35, 64, FAKE, FAKE), cm.ERR_INVALID_ARG),
    ((FAKE + 8, 4, 8, FAKE, FAKE), cm.ERR_ALIGNMENT),
    ((FAKE, 4, 8, FAKE + 4, FAKE), cm.ERR_ALIGNMENT),
    ((FAKE, 4, 8, FAKE, FAKE + 2), cm.ERR_ALIGNMENT),
])
def test_quantize_fp8_rejects_bad_arguments(args, status):
    assert cm.colibri_moe_quantize_fp8(*args) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE + 4096, 64), cm.ERR_INVALID_ARG),
    ((FAKE, None, 64), cm.ERR_INVALID_ARG),
    ((FAKE, FAKE + 4096, 0), cm.ERR_INVALID_ARG),
    ((FAKE, FAKE + 4096, 24), cm.ERR_INVALID_ARG),
    ((FAKE, FAKE + 32, 64), cm.ERR_INVALID_ARG),   # overlapping ranges
    ((FAKE + 32, FAKE, 64), cm.ERR_INVALID_ARG),
    ((FAKE + 8, FAKE + 4096, 64), cm.ERR_ALIGNMENT),
    ((FAKE, FAKE + 4100, 64), cm.ERR_ALIGNMENT),
])
def test_stream_copy_rejects_bad_arguments(args, status):
    # Checked before anything reaches the device (no GPU here).
    assert cm.colibri_moe_stream_copy(*args) == status
