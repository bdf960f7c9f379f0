"""Helpers shared by the GPU parity tests: put seeded inputs on the GPU, run
the library through its C ABI, and compare every graded output with the CPU
oracle.

Comparison rules (all written here, in the tests; "near tie" as decided by
oracle.near_tie_tokens / oracle.boundary_tie_tokens, pinned in
test_oracle_ties.py):
  * logits:   |gpu - ref| <= 1e-5 * max(1, |ref|)
  * ids:      bit-exact on every token whose sorted oracle logits have no
              adjacent pair among the first k+1 closer than 1e-5 relative.
              Near ties inside the top k (not at the k-th / (k+1)-th pair):
              the same set of experts, matched by expert id, in an order the
              oracle's logits allow (each slot's logit at least the next
              one's, up to the tie tolerance). Near ties at the boundary: k
              distinct experts, none of whose oracle logits is below an
              unselected expert's by more than the tie tolerance, in an order
              the logits allow.
  * weights:  on every token, |gpu - ref| <= 1e-5 where ref is the oracle's
              softmax over the logits of the experts the GPU selected, in the
              GPU's slot order (on tokens without near ties that is the
              oracle's own top-k weights).
  * dispatch: counts, offsets, perm, perm_slot and inv bit-exact against the
              oracle's stable counting sort applied to the GPU's own ids (and,
              when no token is near-tied, to the oracle's ids).
  * y:        per-token norm-wise error max_o |y - y_ref| / max_o |y_ref| at
              most 1e-4 (fp32 layers) or 2e-2 (bf16 layers) on every token,
              y_ref from the oracle run with the GPU's ids (identical to the
              oracle's own ids on every token that is not a near tie).
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL_Y = {"f32": 1e-4, "bf16": 2e-2}
TOL_LOGIT_REL = 1e-5
TOL_W = 1e-5


def to_dev(a: np.ndarray):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda")


def to_f64(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def make_layer(cfg: synth.LayerConfig, inp: dict, max_tokens: int | None = None, flags: int = 0):
    import sparse_moe_gemm_amd as cm

    return cm.MoELayer(to_dev(inp["w_router"]), to_dev(inp["b_router"]), to_dev(inp["w_gate"]),
                       to_dev(inp["w_up"]), to_dev(inp["w_down"]), cfg.k,
                       max_tokens=max_tokens or max(cfg.T, 1), flags=flags)


def run_gpu(layer, x: np.ndarray) -> dict:
    import torch

    T = x.shape[0]
    rt = layer.routing_buffers(T)
    y = layer.forward(to_dev(x), routing=rt)
    torch.cuda.synchronize()
    out = {n: v.cpu().numpy() for n, v in rt.items()}
    out["y"] = to_f64(y)
    return out


def compare(cfg: synth.LayerConfig, inp: dict, g: dict, tokens: np.ndarray | None = None,
            ref_layer: oracle.Layer | None = None, act_fp8: bool = False, tol_y: float | None = None) -> dict:
    """Assert every rule in the module docstring; returns a small report.
    act_fp8: the reference y is the oracle's 8-bit activation mode; tol_y
    replaces the dtype's per-token y tolerance."""
    x = inp["x"]
    T, k, E = x.shape[0], cfg.k, cfg.E
    L = ref_layer or oracle.Layer.from_inputs(inp, k)
    lg_ref = L.router(x)
    lg = g["logits"]
    bad = np.abs(lg.astype(np.float64) - lg_ref) > TOL_LOGIT_REL * np.maximum(1.0, np.abs(lg_ref))
    assert not bad.any(), f"logits differ at {np.argwhere(bad)[:5].tolist()}"

    ids_ref, w_ref, _ = oracle.topk(lg_ref, k)
    gid = g["topk_ids"]
    near = oracle.near_tie_tokens(lg_ref, k)
    bnd = oracle.boundary_tie_tokens(lg_ref, k)
    mism = np.where(~near & np.any(gid != ids_ref, axis=1))[0]
    assert mism.size == 0, f"ids differ on tokens {mism[:8].tolist()}"
    for t in np.where(near)[0]:
        sel = gid[t].tolist()
        assert len(set(sel)) == k and all(0 <= e < E for e in sel), f"invalid ids at token {t}: {sel}"
        if not bnd[t]:
            assert sorted(sel) == sorted(ids_ref[t].tolist()), f"id set differs at token {t}"
        lt = lg_ref[t].astype(np.float64)
        tol = lambda a, b: TOL_LOGIT_REL * max(abs(a), abs(b))  # noqa: E731
        for j in range(k - 1):  # slot order allowed by the logits
            a, b = lt[sel[j]], lt[sel[j + 1]]
            assert a >= b - tol(a, b), f"slot order at token {t}"
        if bnd[t]:  # no unselected expert clearly above a selected one
            lo = min(lt[e] for e in sel)
            hi = max((lt[e] for e in range(E) if e not in sel), default=-np.inf)
            assert lo >= hi - tol(lo, hi), f"selection at token {t}"
    w_of_gpu_ids, _ = oracle.route_weights(lg_ref, gid)
    dw = np.abs(g["topk_w"].astype(np.float64) - w_of_gpu_ids.astype(np.float64))
    assert dw.size == 0 or dw.max() <= TOL_W, f"weights differ by {dw.max():.3e}"
    assert np.array_equal(w_of_gpu_ids[~near], w_ref[~near])

    d_gpu_ids = oracle.dispatch(g["topk_ids"], E)
    for key, gk in (("counts", "expert_counts"), ("offsets", "expert_offsets"), ("perm", "perm"),
                    ("perm_slot", "perm_slot"), ("inv", "inv")):
        assert np.array_equal(g[gk], d_gpu_ids[key]), f"dispatch {key} differs"
    if not near.any():
        d_ref = oracle.dispatch(ids_ref, E)
        assert np.array_equal(g["perm"], d_ref["perm"]) and np.array_equal(g["expert_counts"], d_ref["counts"])

    toks = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    y_ref = L.forward(x, tokens=toks, forced_ids=g["topk_ids"], act_fp8=act_fp8)
    y = g["y"][toks]
    den = np.max(np.abs(y_ref), axis=1)
    err = np.max(np.abs(y - y_ref), axis=1) / np.where(den > 0, den, 1.0)
    tol = TOL_Y[cfg.dtype] if tol_y is None else tol_y
    worst = int(np.argmax(err))
    assert err.max() <= tol, f"y per-token error {err.max():.3e} > {tol} at token {toks[worst]}"
    return dict(max_err=float(err.max()), mean_err=float(err.mean()), over_2e2=int((err > 2e-2).sum()),
                near_ties=int(near.sum()), tokens_checked=int(toks.size),
                empty_experts=int((g["expert_counts"] == 0).sum()))
