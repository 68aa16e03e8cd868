"""Helpers shared by the GPU parity tests (no kernels of their own)."""
import sys

import numpy as np
import torch

import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import workloads as W

# Tolerances of the layer's float outputs (relative L2 over a whole output):
# fp32 weights and tokens 1e-5; bf16 or int4 weights 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2, "int4g128": 2e-2, "int4g128_resplit": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def host_weights(shape, blob, shared=False):
    fn = W.shared_expert_weights if shared else W.expert_weights
    return {k: v.cpu() for k, v in fn(shape, blob, device="cuda").items()}


_SPLIT_CACHE: dict = {}


def split_weights(shape, blob, shared=False):
    """The oracle's split-precision parts (O.resplit_expert) of a weight set's fp32 masters."""
    key = (shape.name, blob, shared)
    if key not in _SPLIT_CACHE:
        w = host_weights(shape, blob, shared)
        _SPLIT_CACHE.clear()  # one set at a time: full-size parts are large
        _SPLIT_CACHE[key] = O.resplit_expert(w["gate"].numpy(), w["up"].numpy(), w["down"].numpy())
    return _SPLIT_CACHE[key]


def oracle_expert(shape, x_rows, blob, critical=True, shared=False):
    """Oracle output of weight set `blob` on x_rows; split-precision experts at W^H
    when critical, else at W^L."""
    if shape.wfmt == "int4g128_resplit":
        return O.swiglu_expert_split(x_rows, split_weights(shape, blob, shared), critical)
    return O.expert_forward(x_rows, host_weights(shape, blob, shared))


def oracle_y_rows(shape, x, ids, perm_np, offsets_np, layer, distinct, critical=None):
    """Oracle expert output per sorted position, [T*k, H] float64. critical: the
    experts run at high precision (split-precision experts; None = all)."""
    k = ids.shape[1]
    x32 = O.as_f32(x)
    y = np.zeros((ids.size, shape.H))
    for e in distinct:
        e = int(e)
        rows = perm_np[offsets_np[e]:offsets_np[e + 1]]
        hi = critical is None or e in critical
        y[offsets_np[e]:offsets_np[e + 1]] = oracle_expert(shape, x32[rows // k],
                                                           W.blob_of(shape, layer, e), hi)
    return y


def check_routing(x, wr, bias, k, logits_g, ids_g, w_g, tau_rel=1e-5):
    """Stage parity of moe_route; returns (n_tokens_under_margin, max logit rel err)."""
    lg = logits_g.cpu().numpy()
    ig = ids_g.cpu().numpy()
    wg = w_g.cpu().numpy()
    ref = O.route(x, wr, bias, k)
    scale = 1.0 + np.abs(ref["logits"]).max(axis=1, keepdims=True)
    err = np.abs(lg.astype(np.float64) - ref["logits"]) / scale
    assert err.max() <= 1e-5, f"logits differ: {err.max()}"
    # (i) selection and weights recomputed from the kernel's own logits: exact ids
    assert np.array_equal(O.select_topk(lg, k), ig)
    np.testing.assert_allclose(wg, O.gate_weights(lg.astype(np.float64), ig), rtol=0, atol=1e-6)
    # (ii) against the oracle's own logits, away from near-ties
    tau = tau_rel * (1.0 + np.abs(ref["logits"]).max(axis=1))
    sure = ref["margin"] > tau
    assert np.array_equal(ig[sure], ref["ids"][sure])
    return int((~sure).sum()), float(err.max())
