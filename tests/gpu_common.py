"""Helpers shared by the GPU parity tests (no kernels of their own)."""
import sys

import numpy as np
import torch

import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import harness as Hn
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


class OracleWeights:
    """Host weights of every weight set the oracle's pool may copy, drawn once each (the
    split-precision parts for split-precision shapes)."""

    def __init__(self, shape):
        self.shape = shape
        self.cache: dict = {}

    def get(self, blob, shared=False):
        key = (blob, shared)
        if key not in self.cache:
            if self.shape.wfmt == "int4g128_resplit":
                w = host_weights(self.shape, blob, shared)
                self.cache[key] = O.resplit_expert(w["gate"].numpy(), w["up"].numpy(), w["down"].numpy())
            else:
                self.cache[key] = host_weights(self.shape, blob, shared)
        return self.cache[key]

    def of(self, layer, expert):
        return self.get(W.blob_of(self.shape, layer, expert))


def run_layer_case(shape, slots, mode, Ts, layers_order=None, policy=None, device_plan=False,
                   split=None, staging=None, sample=None, weights=None):
    """Run steps through the runtime and compare every step with the oracle's layer
    (O.moe_layer over its own slot pool and planner, the weights read through the pool).

    Routing: stage parity on the kernel's logits and margin-gated ids (check_routing); the
    oracle routes on its own logits. Tables: the runtime's lut, last use and clock equal the
    oracle planner's after every step. Output: relative L2 over the tokens whose ids agree
    (all tokens but near-ties), within the format's tolerance.
    policy = (kind, window, params): the runtime plans under that eviction policy and the
    oracle's scored planner takes the kernel's step scores (checked against the oracle's
    softmax of the kernel's logits). device_plan: the runtime plans and fills on the GPU.
    split = (theta, beta, gamma): split-precision routing; the oracle takes the critical set
    from the kernel's step scores in float32.
    staging = token threshold: steps of layers not wholly resident with T >= threshold run
    from the full-layer staging buffers; the oracle reads that layer from a pool holding all
    of its experts and its planner (the decode cache) skips the step.
    sample(T, ids) -> token rows whose outputs the oracle computes (None: all).
    Returns the layer object."""
    t_max = max(Ts)
    residency = W.initial_residency(shape, slots, mode)
    layer_obj = Hn.SlotCacheLayer(shape, slots, residency, t_max, staging=staging is not None)
    if staging is not None:
        layer_obj.ctx.set_staging(True, staging)
    if device_plan:
        layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    if split is not None:
        theta, beta, gamma = split
        layer_obj.ctx.set_split(True, theta, beta, gamma)
    wts_src = weights or OracleWeights(shape)
    pool = O.SlotPool(slots, shape.layers, shape.E)
    for s_, o_ in enumerate(residency):
        if o_ is not None:
            pool.commit(s_, o_[0], o_[1], wts_src.of(*o_))
    shared = [wts_src.get(j, shared=True) for j in range(shape.n_shared)]
    n_hi = n_lo = 0
    if policy is None:
        planner = O.LruSlotPlanner(slots, shape.layers, shape.E, residency)
    else:
        kind, window, params = policy
        layer_obj.ctx.set_policy(kind, window, params)
        pol = (O.MinusRecentScore(shape.layers, shape.E, window) if kind == B.MOE_POLICY_MRS else
               O.RoutingHistoryScore(shape.layers, shape.E, window, weights=params[:4], lam=params[4]))
        planner = O.ScoredSlotPlanner(slots, shape.layers, shape.E, pol, residency)
    order = layers_order or [0]
    for step, T in enumerate(Ts):
        for layer in order:
            say(f"layer {shape.name} step={step} layer={layer} T={T}")
            x = W.tokens(shape, T, layer=layer, step=step, device="cuda")
            out = layer_obj.forward(x, layer=layer)
            torch.cuda.synchronize()
            assert layer_obj.err.item() == 0
            wr, b = layer_obj.routers[layer]
            o = layer_obj.outputs(T)
            under, _ = check_routing(x, wr, b, shape.k, o["logits"], o["ids"], o["topk_w"])
            ids = o["ids"].cpu().numpy()
            pr = O.permute(ids, shape.E)
            assert o["perm"].cpu().numpy().tolist() == pr["perm"].tolist()
            assert o["inv"].cpu().numpy().tolist() == pr["inv"].tolist()
            sc = None
            if policy is not None or split is not None:
                sc = layer_obj.ctx.step_scores()
                np.testing.assert_allclose(sc, O.step_scores(o["logits"].cpu().numpy()), rtol=2e-6, atol=1e-7)
            n_res = int(np.sum(planner.lut[layer] >= 0))
            staged = (staging is not None and n_res < shape.E
                      and T >= (staging if staging >= 0 else n_res // shape.k))
            crit = None
            if split is not None:
                th = O.critical_threshold(theta, 1.0 if beta is None else beta[layer], "decode", gamma)
                crit = set(O.critical_experts(sc, pr["distinct"], th))
                n_hi += len(crit)
                n_lo += len(pr["distinct"]) - len(crit)
            # the sample is chosen on the oracle's own routing
            rows = None if sample is None else sample(T, O.route(x, wr, b, shape.k)["ids"])
            if staged:  # the layer's own full buffer; the decode cache is not touched
                spool = O.SlotPool(shape.E, shape.layers, shape.E)
                for e in range(shape.E):
                    spool.commit(e, layer, e, wts_src.of(layer, e))
                ref = O.moe_layer(x, wr, b, shape.k, layer=layer, pool=spool, planner=None,
                                  weights_of_expert=lambda e, l=layer: wts_src.of(l, e), shared=shared,
                                  critical=crit, rows=rows)
            else:
                ref = O.moe_layer(x, wr, b, shape.k, layer=layer, pool=pool, planner=planner,
                                  weights_of_expert=lambda e, l=layer: wts_src.of(l, e), shared=shared,
                                  scores=sc if policy is not None else None, critical=crit, rows=rows)
            assert np.array_equal(ref["perm"]["distinct"], pr["distinct"]), "routed sets differ"
            lut_h, owner_h, last_use_h, clock_h = layer_obj.tables()
            assert layer_obj.lut.cpu().numpy().reshape(shape.layers, shape.E).tolist() == planner.lut.tolist()
            assert lut_h.reshape(shape.layers, shape.E).tolist() == planner.lut.tolist()
            assert last_use_h.tolist() == planner.last_use and clock_h == planner.clock
            same = np.all(ref["route"]["ids"] == ids, axis=1)
            keep = same if rows is None else same & np.isin(np.arange(T), rows)
            got = out.float().cpu().numpy()
            r = rel_l2(got[keep], ref["out"][keep])
            cnt = layer_obj.counters()
            say(f"  rel L2 {r:.3e} over {int(keep.sum())} tokens ({int((~same).sum())} near-tie "
                f"tokens routed differently, {under} under the margin); totals so far {cnt}" +
                (f"; critical {sorted(crit)}" if crit is not None else ""))
            assert r <= TOL[shape.wfmt]
    if split is not None:
        assert n_hi > 0 and n_lo > 0, (n_hi, n_lo)  # both precisions were exercised
    return layer_obj
