"""Benchmark of the routed-expert MoE layer over a device-resident slot cache (one MI355X).

A step is one pass of the whole layer (route, permute, slot lookup and
residency plan, expert FFN over resident slots with fills of the misses,
shared experts, combine) over one batch of synthetic tokens already in HBM;
for the 48-layer stack a step runs every layer once.

Default workload: the largest layer that fits one GPU, DeepSeek-V3-shaped with
int4 weights (256 routed experts, top-8, one shared expert, hidden 7168, expert
FFN 2048 SwiGLU, symmetric int4 codes with one bf16 scale per 128 inputs) and
int8 per-token activations.

  value     decode, 1 token per step, through the workload's own cache of 84 slots
            (Zipf(1.1) routing, initial residency by Zipf rank): misses copied from
            pinned host memory over PCIe on the side stream, victims by HybriMoE's
            Minus Recent Score, tokens/s over the --steps timed steps.
  also      the hit path (every routed expert of the step resident) at 1, 32 and
            4096 tokens (prefill: MFMA share of the int8 peak next to the HBM one);
            a decode step's weights (about 205 MB) fit the 256 MB MALL, so the timed
            steps rotate over replicas of the slot pool and no step finds its
            weights left in the MALL by the previous one; the cache with fills at
            1 and 32 tokens under each eviction policy; the other four workloads'
            hit paths and caches.
  roofline  the expert FFN stage of the same shape and token count on the hit
            path (one moe_expert_ffn call: gate/up pass + down pass): algorithmic
            bytes (weights of the distinct routed experts and the shared one +
            tokens in + rows out) per call divided by its HIP-event duration on the
            compute stream.
  cpu_baseline  the oracle (float64 NumPy) on a bounded sample of the headline's
            decode steps, on every core the process may use.

Other workloads (--workload NAME) print a line of the same form for that
workload. --case runs one case without a JSON line (profiling).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload NAME] [--quick] [--case CASE]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from expert_offload_routed_amd import binding as B  # noqa: E402
from expert_offload_routed_amd import harness as Hn  # noqa: E402
from expert_offload_routed_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "int4g128": 5000.0, "f32": 157.3}  # dense; int8 ops for int4 weights
DEFAULT = "dsv3_e256k8s1_h7168_f2048_int4"
METRIC = "MoE-layer tokens/s at 1 GPU + achieved HBM GB/s (decode) / MFMA % (prefill)"


def expert_bytes(shape) -> int:
    H, F = shape.H, shape.F
    if shape.is_int4:  # codes, plus one bf16 scale per 128 weights
        return 3 * H * F // 2 + 3 * (H * F // 128) * 2
    return 3 * H * F * {"f32": 4, "bf16": 2}[shape.wfmt]


def _xbytes(shape) -> int:
    return 4 if shape.xfmt == "f32" else 2


def _run(layers, batches, out, timing):
    """batches: list of steps, each a list of (layer index, x); step i runs on
    layers[i % len(layers)] (replicas of one slot pool, see timed)."""
    for lay in layers:
        lay.ctx.set_timing(timing)
    c0 = [lay.counters() for lay in layers]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, step in enumerate(batches):
        lay = layers[i % len(layers)]
        if len(step) == 1:
            lay.forward(step[0][1], layer=step[0][0], out=out)
        else:  # a stack step: every layer in one native call
            lay.forward_steps(step, out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    cnt = {}
    ms = n = 0
    for lay, a in zip(layers, c0):
        b = lay.counters()
        for k in b:
            cnt[k] = cnt.get(k, 0) + b[k] - a[k]
        m, c = lay.ctx.ffn_time()
        ms, n = ms + m, n + c
        lay.ctx.set_timing(False)
    return dt, cnt, ms, n


def make_batches(shape, T, steps, layer_rho=None):
    """steps x layers token batches: independent draws, or AR(1) per layer for a stack.

    layer_rho (stack only): chain the layers' inputs as a stand-in for a residual stream,
    x[l+1] = rho x[l] + sqrt(1 - rho^2) e[l+1], where e[l] is layer l's own AR(1) input, so
    that layer l's tokens carry information about layer l+1's routing."""
    if shape.layers == 1:
        return [[(0, W.tokens(shape, T, step=i, device="cuda"))] for i in range(steps)]
    seqs = [W.token_sequence(shape, T, steps, layer=l, device="cuda") for l in range(shape.layers)]
    if layer_rho is not None:
        c = float(np.sqrt(1.0 - layer_rho * layer_rho))
        for l in range(1, shape.layers):
            seqs[l] = (layer_rho * seqs[l - 1].float() + c * seqs[l].float()).to(seqs[l].dtype)
    return [[(l, seqs[l][i]) for l in range(shape.layers)] for i in range(steps)]


def timed(layers, shape, T, steps, warmup, label, ffn_timing=False, layer_rho=None):
    """Warm up, then time exactly ``steps`` steps between two device synchronisations.

    layers: one layer object, or replicas of it (each its own slot pool holding the
    same experts) that the steps use in turn, so that a step's weights were last read
    several steps earlier. With ffn_timing, the same steps run a second time with HIP
    events on the compute stream around each layer call's expert FFN (routed groups,
    fill waves, shared experts); the headline rate comes from the pass without events.
    """
    layers = layers if isinstance(layers, (list, tuple)) else [layers]
    batches = make_batches(shape, T, steps + warmup, layer_rho)
    out = torch.empty(T, shape.H, dtype=layers[0].out_dtype, device="cuda")
    _run(layers, batches[:warmup], out, False)
    dt, cnt, _, _ = _run(layers, batches[warmup:], out, False)
    calls = steps * shape.layers
    res = {"tokens_per_step": T, "tokens_per_s": steps * T / dt, "ms_per_step": dt / steps * 1e3,
           "distinct_per_layer_call": cnt["distinct"] / calls,
           "fills_per_step": cnt["fills"] / steps, "pool_replicas": len(layers)}
    if cnt["distinct"] > 0:
        res["hit_rate"] = cnt["hits"] / cnt["distinct"]
    if ffn_timing:
        dt2, cnt2, ms, n = _run(layers, batches[warmup:], out, True)
        eb = expert_bytes(shape)
        # algorithmic bytes of the expert FFN per layer call: each distinct routed
        # expert's weights once, the shared experts' weights, tokens in, fp32 rows out
        per_call = (cnt2["distinct"] / calls) * eb + shape.n_shared * eb + T * shape.H * _xbytes(shape) \
            + T * (shape.k + shape.n_shared) * shape.H * 4
        flops = 6.0 * T * (shape.k + shape.n_shared) * shape.H * shape.F
        us = 1e3 * ms / n
        res["ffn"] = {"calls": n, "avg_us": us, "bytes_per_call": per_call,
                      "gbs": per_call / (us * 1e-6) / 1e9,
                      "mfma_frac": flops / (us * 1e-6) / (MFMA_PEAK_TFLOPS[shape.wfmt] * 1e12),
                      "ms_per_step_with_events": dt2 / steps * 1e3}
    print(f"# {shape.name} {label}: {res}", file=sys.stderr, flush=True)
    return res


def replicas_for(shape, T, max_bytes=24e9):
    """Pool replicas a hit-path timing rotates over: enough that the weights of the
    steps in between exceed 1 GB (four times the 256 MB MALL), at most 8 and at most
    max_bytes of pools. The 48-layer stack reads GBs per step: one pool."""
    if shape.layers > 1:
        return 1
    p = 1.0 - (1.0 - 1.0 / shape.E) ** (T * shape.k)  # chance that an expert is routed
    per_step = (shape.E * p + shape.n_shared) * expert_bytes(shape)
    pool = (shape.E + shape.n_shared) * expert_bytes(shape)
    r = int(np.ceil(1e9 / per_step)) + 1 if per_step < 1e9 else 1
    return max(1, min(8, r, int(max_bytes // pool)))


def recorded_traffic(*keys):
    """HBM bytes per FFN call (FETCH_SIZE + WRITE_SIZE runs, calibrated), as recorded in
    profiles/ffn_traffic.json under the first of keys present; None when absent or when an
    FFN kernel source changed since."""
    try:
        recs = json.load(open(os.path.join(ROOT, "profiles", "ffn_traffic.json")))
    except (OSError, ValueError):
        return None
    rec = next((recs[k] for k in keys if k in recs), None)
    if rec is None:
        return None
    return rec["read_bytes"] + rec["write_bytes"] if ffn_sources_sha1() == rec["csrc_sha1"] else None


# the sources the expert-FFN kernels are compiled from (routing, runtime and combine excluded)
FFN_SOURCES = ("common.h", "ffn_internal.h", "ffn.hip", "ffn_gemv.h", "tile_gemv.h", "gemm.hip",
               "skinny.hip", "ffn_int4.hip", "decode_share.h", "decode_int4.hip", "decode_bf16.hip")


def ffn_sources_sha1() -> str:
    import hashlib
    h = hashlib.sha1()
    for name in FFN_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(ROOT, "expert_offload_routed_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def all_resident(shape):
    """Every layer-expert in its own slot, in a seeded random slot order."""
    own = [(l, e) for l in range(shape.layers) for e in range(shape.E)]
    rng = np.random.Generator(np.random.PCG64(W.seed_for(shape, "residency", len(own), 1)))
    return [own[i] for i in rng.permutation(len(own))]


def cpu_baseline(shape, budget_s=20.0):
    """The oracle as it stands (float64 NumPy), on a bounded sample of the headline's decode
    steps (1 token per step, layer 0, every routed expert resident in the oracle's pool), on
    every core the process may use (BLAS threads set to that count, capped by the thread
    budget the environment sets)."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    affinity = len(os.sched_getaffinity(0))
    env_cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(affinity, env_cap) if env_cap > 0 else affinity
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    E = shape.E
    cache = {}
    load_s = [0.0]  # drawing the synthetic weights is setup, not oracle work: not counted

    def weights_of(e):
        if e not in cache:
            t = time.perf_counter()
            cache[e] = {n: v.cpu() for n, v in
                        W.expert_weights(shape, W.blob_of(shape, 0, e), device="cuda").items()}
            load_s[0] += time.perf_counter() - t
        return cache[e]

    shared = [{n: t.cpu() for n, t in W.shared_expert_weights(shape, j, device="cuda").items()}
              for j in range(shape.n_shared)]
    wr, b = W.router(shape)
    # the oracle's pool of E slots starts empty: an expert is copied in on its first use
    pool = O.SlotPool(E, 1, E)
    planner = O.LruSlotPlanner(E, 1, E, [None] * E)
    n, work = 0, 0.0
    with threadpool_limits(limits=threads):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        while True:
            x = W.tokens(shape, 1, step=n)
            t0, l0 = time.perf_counter(), load_s[0]
            O.moe_layer(x, wr, b, shape.k, layer=0, pool=pool, planner=planner,
                        weights_of_expert=weights_of, shared=shared or None)
            work += time.perf_counter() - t0 - (load_s[0] - l0)
            n += 1
            if work >= budget_s or n >= 64:
                break
    return {"value": n / work, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{n} decode steps of 1 token of {shape.name}, layer 0 (float64 NumPy oracle, "
                      f"int4 weights dequantised per use), {work:.1f} s of oracle time",
            "affinity_cores": affinity, "cpu_model": model}


def cpu_baseline_tiny(budget_s=3.0):
    """The oracle on the tiny fp32 layer (16 tokens per step, every expert resident in its
    pool) on one thread: the single-core reference the parity configuration is timed at."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    shape = W.shape_of("tiny_e8k2_h256_f512_fp32")
    E, T = shape.E, 16
    weights = {e: W.expert_weights(shape, W.blob_of(shape, 0, e)) for e in range(E)}
    wr, b = W.router(shape)
    pool = O.SlotPool(E, 1, E)
    planner = O.LruSlotPlanner(E, 1, E, [None] * E)
    n, work = 0, 0.0
    with threadpool_limits(limits=1):
        while work < budget_s and n < 4096:
            x = W.tokens(shape, T, step=n)
            t0 = time.perf_counter()
            O.moe_layer(x, wr, b, shape.k, layer=0, pool=pool, planner=planner,
                        weights_of_expert=lambda e: weights[e])
            work += time.perf_counter() - t0
            n += 1
    return {"value": n * T / work, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} steps of {T} tokens of {shape.name} (float64 NumPy oracle), "
                      f"{work:.1f} s on one thread"}


def calib_copy(steps):
    """Plain device copy of 1 GiB, for scaling the HBM byte counters (FETCH_SIZE, WRITE_SIZE)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(f"# copy 1 GiB x {steps}: {2 * n * steps / dt / 1e9:.1f} GB/s (read + write)", file=sys.stderr)


# token counts timed per workload (hit path) and the caches with fills
PLANS = {
    "tiny_e8k2_h256_f512_fp32": dict(hit=[16], miss=[]),
    "mixtral_e8k2_h4096_f14336_bf16": dict(hit=[1, 8, 512], miss=[(4, 1)]),
    "qwen3moe_l48_e128k8_h2048_f768_bf16": dict(hit=[1, 16], miss=[(2765, 1), (2765, 16)]),
    "dsv2lite_e64k6s2_h2048_f1408_bf16": dict(hit=[1, 32, 256, 1024], miss=[(16, 1), (32, 1), (48, 1)]),
    "dsv3_e256k8s1_h7168_f2048_int4": dict(hit=[1, 32, 4096], miss=[(84, 1), (84, 32)]),
}
CASES = {"decode1": 1, "decode8": 8, "prefill512": 512}
# eviction policies compared on the caches with fills: (kind, window, params). The pages give
# no window, weights or decay; these are the readings (window of 8 steps, equal weights, 0.9).
# "*_device": the same plan run by the GPU itself (device orchestration, no host wait).
POLICIES = {"lru": (B.MOE_POLICY_LRU, 1, None),
            "mrs": (B.MOE_POLICY_MRS, 8, None),
            "history": (B.MOE_POLICY_HISTORY, 8, [1.0, 1.0, 1.0, 1.0, 0.9]),
            "lru_device": (B.MOE_POLICY_LRU, 1, None),
            "mrs_device": (B.MOE_POLICY_MRS, 8, None),
            "history_device": (B.MOE_POLICY_HISTORY, 8, [1.0, 1.0, 1.0, 1.0, 0.9])}


def fill_cases(shape, plan, cfg, store, steps, warmup, policies=tuple(POLICIES), head=None):
    """Each cache with fills of the workload under each of the eviction policies named, on
    the same inputs (rates include the PCIe copies of the misses). head = (steps, warmup):
    the first cache under HEAD_POLICY runs that many steps instead (the headline)."""
    out = {}
    for ci, (S, T) in enumerate(plan["miss"]):
        res = {}
        for name in policies:
            n_steps, n_warm = (head if head is not None and ci == 0 and name == HEAD_POLICY
                               else (steps, warmup))
            kind, window, params = POLICIES[name]
            small = Hn.SlotCacheLayer(shape, S, W.initial_residency(shape, S, cfg["residency"]),
                                      t_max=T, store=store)
            small.ctx.set_policy(kind, window, params)
            if name.endswith("_device"):
                if T * shape.k > S:
                    continue  # more routed experts than slots: only the host plans it
                small.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
            r = timed(small, shape, T, n_steps, n_warm,
                      f"T={T}, {S} slots ({cfg['residency']}), {name} eviction, fills over PCIe")
            r["fill_bytes_per_step"] = r["fills_per_step"] * store.stride
            res[name] = r
            del small
            torch.cuda.empty_cache()
        out[f"T{T}_{S}slots_with_fills"] = res
    return out


def graph_case(shape, plan, cfg, store, steps, warmup):
    """Every cache with fills under device orchestration, eager and as one captured HIP graph
    per stack step (inputs for each step copied into the graph's static input buffer with one
    copy, inside the timed region)."""
    for S, T in plan["miss"]:
        if T * shape.k > S:
            continue
        for graphed in (False, True):
            s = torch.cuda.Stream()
            lay = Hn.SlotCacheLayer(shape, S, W.initial_residency(shape, S, cfg["residency"]), t_max=T,
                                    store=store, compute_stream=s)
            lay.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
            batches = make_batches(shape, T, steps + warmup)
            X = torch.stack([torch.stack([x for _, x in b]) for b in batches])  # [steps, L, T, H]
            xin = torch.empty_like(X[0])
            outs = [torch.empty(T, shape.H, dtype=lay.out_dtype, device="cuda") for _ in range(shape.layers)]

            def step():
                for l in range(shape.layers):
                    lay.forward(xin[l], layer=l, out=outs[l])

            g = None
            with torch.cuda.stream(s):
                for i in range(warmup):
                    xin.copy_(X[i])
                    step()
            torch.cuda.synchronize()
            if graphed:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step()
                torch.cuda.synchronize()
            c0 = lay.counters()
            t0 = time.perf_counter()
            with torch.cuda.stream(s):
                for i in range(warmup, warmup + steps):
                    xin.copy_(X[i])
                    g.replay() if graphed else step()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            c1 = lay.counters()
            res = {"tokens_per_s": steps * T / dt, "ms_per_step": dt / steps * 1e3,
                   "fills_per_step": (c1["fills"] - c0["fills"]) / steps,
                   "hit_rate": (c1["hits"] - c0["hits"]) / max(1, c1["distinct"] - c0["distinct"])}
            print(f"# T={T}, {S} slots, device orchestration, {'graph' if graphed else 'eager'}: {res}",
                  file=sys.stderr, flush=True)
            del lay, g
            torch.cuda.empty_cache()


def split_bytes(shape) -> tuple[int, int]:
    """Algorithmic bytes one split-precision expert streams at low (W^L: int4 gate/up/down) and
    at high precision (W^H: int4 gate/up and their int4 residual, 8-bit down), scales included."""
    H, F = shape.H, shape.F
    s13, s2 = 2 * F * (H // 128) * 2, H * (F // 128) * 2
    low = 2 * F * H // 2 + s13 + H * F // 2 + s2
    high = 2 * (2 * F * H // 2 + s13) + H * F + s2
    return low, high


def split_case(shape, store, T, steps, warmup, critical_share=0.25):
    """Split-precision routing on the hit path (every expert resident): every routed expert at
    low precision, the split (theta set so that about `critical_share` of the routed experts of
    the calibration steps are critical), and every expert at high precision. For each: tokens/s,
    the expert FFN's HIP-event time and its algorithmic bytes from the counted critical groups."""
    layer = Hn.SlotCacheLayer(shape, shape.E, all_resident(shape), t_max=T, store=store)
    batches = make_batches(shape, T, steps + warmup)
    out = torch.empty(T, shape.H, dtype=layer.out_dtype, device="cuda")
    # calibration: the routed experts' scores over the warm-up batches
    layer.ctx.set_split(True, 0.0)
    routed_scores = []
    for b in batches[:warmup]:
        layer.forward(b[0][1], out=out)
        sc = layer.ctx.step_scores()
        ids = np.unique(layer.outputs(T)["ids"].cpu().numpy())
        routed_scores += sc[ids].tolist()
    theta = float(np.quantile(routed_scores, 1.0 - critical_share))
    low_b, high_b = split_bytes(shape)
    res = {"theta": theta, "expert_bytes_low": low_b, "expert_bytes_high": high_b}
    for mode, th in (("all_low", float("inf")), ("split", theta), ("all_high", 0.0)):
        if np.isinf(th):
            layer.ctx.set_split(True, 3.0e38)
        else:
            layer.ctx.set_split(True, th)
        _run(layer, batches[:warmup], out, False)
        dt, _, _, _ = _run(layer, batches[warmup:], out, False)
        _, _, ms, n = _run(layer, batches[warmup:], out, True)
        # critical groups per step, counted on the same batches (one host read per step)
        n_hi = n_lo = 0
        for b in batches[warmup:]:
            layer.forward(b[0][1], out=out)
            sc = layer.ctx.step_scores()
            ids = np.unique(layer.outputs(T)["ids"].cpu().numpy())
            hi = int(np.sum(sc[ids] >= np.float32(3.0e38 if np.isinf(th) else th)))
            n_hi += hi
            n_lo += len(ids) - hi
        us = 1e3 * ms / n
        per_call = (n_lo * low_b + n_hi * high_b) / steps + shape.n_shared * high_b \
            + T * shape.H * _xbytes(shape) + T * (shape.k + shape.n_shared) * shape.H * 4
        r = {"tokens_per_s": steps * T / dt, "ms_per_step": dt / steps * 1e3,
             "critical_per_step": n_hi / steps, "low_per_step": n_lo / steps,
             "ffn": {"avg_us": us, "bytes_per_call": per_call, "gbs": per_call / (us * 1e-6) / 1e9}}
        print(f"# T={T} split precision, {mode}: {r}", file=sys.stderr, flush=True)
        res[mode] = r
    del layer
    torch.cuda.empty_cache()
    return res


def staging_case(shape, cfg, store, S, T, steps, warmup):
    """Prefill of T tokens per layer through the workload's own cache (S slots): the decode
    cache alone (misses filled in waves), then with full-layer staging at the pages' switch
    floor(resident slots of the layer / k), the next layer loading while one computes."""
    res = {}
    for staged in (False, True):
        lay = Hn.SlotCacheLayer(shape, S, W.initial_residency(shape, S, cfg["residency"]), t_max=T,
                                store=store, staging=staged)
        if staged:
            lay.ctx.set_staging(True, -1)
        s0 = lay.ctx.stage_counters()
        label = f"T={T} prefill, {S} slots, " + ("full-layer staging" if staged else "decode cache only")
        r = timed(lay, shape, T, steps, warmup, label)
        s1 = lay.ctx.stage_counters()
        # staged steps of the timed region only: warm-up steps are counted before it
        r["stage"] = {k: s1[k] - s0[k] for k in s1}
        r["copy_bytes_per_step"] = (r["fills_per_step"] * store.stride
                                    + (s1["stage_copies"] - s0["stage_copies"]) / (steps + warmup)
                                    * store.stride)
        print(f"# {label}: copies {r['copy_bytes_per_step'] / 1e9:.2f} GB/step, {r['stage']}",
              file=sys.stderr, flush=True)
        res["staging" if staged else "decode_cache"] = r
        del lay
        torch.cuda.empty_cache()
    return res


def hit_layers(shape, T, store, t_max=None):
    """Hit-path layer objects (every layer-expert resident), replicated per replicas_for."""
    resident = all_resident(shape)
    n = replicas_for(shape, T)
    return [Hn.SlotCacheLayer(shape, len(resident), resident, t_max=t_max or T, store=store)
            for _ in range(n)]


# the eviction policy of the headline's cache with fills: HybriMoE's Minus Recent Score, the
# one with the fewest fills on the DeepSeek-V3-shaped decode cache (40 steps at T = 1: 1.2
# fills per step against 1.6 under LRU and 1.475 under the routing-history score; 1,743
# against 1,395 tokens/s with both planned on the GPU)
HEAD_POLICY = "mrs_device"
POLICY_DESC = {"lru": "LRU eviction planned on the host", "lru_device": "LRU eviction planned on the GPU",
               "mrs": "Minus Recent Score eviction (window 8) planned on the host",
               "mrs_device": "Minus Recent Score eviction (window 8) planned on the GPU",
               "history": "routing-history eviction planned on the host",
               "history_device": "routing-history eviction planned on the GPU"}


def pcie_copy(store, n=10) -> dict:
    """One expert's bytes copied from the pinned host store into device memory on a side
    stream (a copy-engine transfer; the fills' copy kernel moves the same 56 GB/s), alone and
    timed with events: the PCIe rate the fills are bound by."""
    dst = torch.empty(store.stride, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nb = store.host.shape[0]
    with torch.cuda.stream(s):
        for i in range(2):
            dst.copy_(store.host[i % nb], non_blocking=True)
        ev0.record(s)
        for i in range(n):
            dst.copy_(store.host[(i + 2) % nb], non_blocking=True)
        ev1.record(s)
    ev1.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / n
    del dst
    return {"bytes": int(store.stride), "us": round(us, 1), "gbs": round(store.stride / us / 1e3, 2)}


def workload_report(name, K, Wm, quick=False, policies=("lru", "lru_device", "mrs", "mrs_device"),
                    head_steps=None):
    """Hit path at each token count of the workload (expert FFN timed with events) and its
    caches with fills (quick: the first hit path and the first cache under HEAD_POLICY).
    Returns (first hit-path result, dict of the others)."""
    shape, plan, cfg = W.shape_of(name), PLANS[name], W.WORKLOADS[name]
    store = Hn.ExpertStore(shape)
    res = {}
    head = None
    for i, T in enumerate(plan["hit"]):
        if quick and i > 0:
            break
        steps = K if T <= 64 else max(K // 10, 3)
        layers = hit_layers(shape, T, store)
        r = timed(layers, shape, T, steps, Wm if i == 0 else 2, f"T={T} hit path", ffn_timing=True)
        del layers
        torch.cuda.empty_cache()
        if head is None:
            head = r
        else:
            res[f"T{T}_hit"] = r
    steps = max(K // 5, 5) if shape.layers == 1 else max(K // 5, 8)
    if plan["miss"]:
        res["pcie_copy"] = pcie_copy(store)
    if not quick:
        res.update(fill_cases(shape, plan, cfg, store, steps, 2, policies, head_steps))
    elif plan["miss"]:
        res.update(fill_cases(shape, dict(plan, miss=plan["miss"][:1]), cfg, store, steps, 2,
                              (HEAD_POLICY,), head_steps))
    del store
    torch.cuda.empty_cache()
    return head, res


def prefetch_case(shape, cfg, store, S, T, steps, warmup, t_remain_us=20.0, t_launch_us=5.0,
                  bw_gbs=55.0, t_attn_list=(0.0, 200.0, 1000.0)):
    """Stack steps through the workload's own cache (S slots), without and with the miss
    prefetch of the next layer (MoE-CORE summary page, Mechanism), for attention times the
    layer itself does not have (the window is t_remain + t_attn - t_launch; the step still
    pays the copies, since no attention runs here to hide them)."""
    res = {}
    for rho, t_attn in [(r_, t_) for r_ in (None, 0.9) for t_ in (None,) + tuple(t_attn_list)]:
        lay = Hn.SlotCacheLayer(shape, S, W.initial_residency(shape, S, cfg["residency"]), t_max=T,
                                store=store)
        if t_attn is not None:
            lay.ctx.set_prefetch(True, t_remain_us, t_attn, t_launch_us, bw_gbs)
        p0 = lay.ctx.prefetch_counters()
        label = ("no prefetch" if t_attn is None else f"prefetch, t_attn = {t_attn:g} us") + \
            ("" if rho is None else f", layer inputs chained (rho {rho:g})")
        r = timed(lay, shape, T, steps, warmup, f"T={T}, {S} slots, {label}", layer_rho=rho)
        p1 = lay.ctx.prefetch_counters()
        r["prefetched_per_step"] = (p1["prefetched"] - p0["prefetched"]) / (steps + warmup)
        r["prefetch_used_per_step"] = (p1["prefetch_used"] - p0["prefetch_used"]) / (steps + warmup)
        if t_attn is not None:
            r["window_us"] = t_remain_us + t_attn - t_launch_us
        print(f"# {label}: prefetched/step {r['prefetched_per_step']:.2f}, used/step "
              f"{r['prefetch_used_per_step']:.2f}", file=sys.stderr, flush=True)
        res[("none" if t_attn is None else f"t_attn_{t_attn:g}us")
            + ("" if rho is None else f"_chained{rho:g}")] = r
        del lay
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(PLANS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline case only")
    ap.add_argument("--case", default=None,
                    help="one case only, for profiling (prints no JSON line): decode1, decode8, "
                         "prefill512, fills, policies (every cache with fills under each eviction "
                         "policy), graph (device orchestration, eager vs one HIP graph per step), "
                         "split (split-precision experts: all low, split, all high; the "
                         "workload's shape with split-precision slots and 16 distinct weight "
                         "sets), staging (prefill through the workload's cache with and without "
                         "full-layer staging), prefetch (stack steps through the workload's cache "
                         "with and without the next layer's miss prefetch), T<n> (hit path at n "
                         "tokens), calib_copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU form of "
              "this layer is a design, not built here.", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    K, Wm = args.steps, args.warmup
    if args.case == "calib_copy":
        calib_copy(K)
        return
    shape = W.shape_of(args.workload)
    plan = PLANS[args.workload]
    cfg = W.WORKLOADS[args.workload]
    if args.case == "staging":
        S = plan["miss"][0][0]
        store = Hn.ExpertStore(shape)
        for T in ([256] if shape.layers > 1 else [max(plan["hit"])]):
            staging_case(shape, cfg, store, S, T, K, Wm)
        return
    if args.case == "prefetch":
        S, T = plan["miss"][0]
        prefetch_case(shape, cfg, Hn.ExpertStore(shape), S, T, K, Wm)
        return
    if args.case == "split":
        # fp32 masters quantised by the library; 16 weight sets back the E slots (each slot
        # its own memory, so the HBM traffic is that of E distinct experts)
        sshape = W.reduced(shape, wfmt="int4g128_resplit", blobs=16, name=shape.name + "_resplit")
        sstore = Hn.ExpertStore(sshape)
        for T in (1, 32, 512):
            split_case(sshape, sstore, T, K if T <= 32 else max(K // 4, 3), Wm)
        return
    if args.case is not None:
        store = Hn.ExpertStore(shape)
        if args.case == "policies":
            fill_cases(shape, plan, cfg, store, K, Wm, tuple(POLICIES))
        elif args.case == "graph":
            graph_case(shape, plan, cfg, store, K, Wm)
        elif args.case == "fills":
            S, T = plan["miss"][0]
            small = Hn.SlotCacheLayer(shape, S, W.initial_residency(shape, S, cfg["residency"]),
                                      t_max=T, store=store)
            timed(small, shape, T, K, Wm, f"T={T}, {S} slots, fills over PCIe")
        else:
            T = CASES[args.case] if args.case in CASES else int(args.case.lstrip("T"))
            timed(hit_layers(shape, T, store), shape, T, K, Wm, args.case, ffn_timing=True)
        return

    hit, also = workload_report(args.workload, K, Wm, args.quick, head_steps=(K, Wm))
    hit_T = plan["hit"][0]
    also = {f"T{hit_T}_hit": hit, **also}
    if not args.quick and args.workload == DEFAULT:
        others = {}
        for name in PLANS:
            if name != DEFAULT:
                h, rest = workload_report(name, max(K // 2, 5), 2)
                others[name] = {f"T{h['tokens_per_step']}_hit": h, **rest}
        also["other_workloads"] = others

    # the headline: the workload's own cache with fills (its first one) under HEAD_POLICY
    # when it has one, else the hit path; the roofline is the expert-FFN stage of the same
    # shape and token count, timed with events on the all-resident steps (same kernels)
    head, head_desc = hit, "every routed expert of the step resident (hit path)"
    if plan["miss"]:
        S0, T0 = plan["miss"][0]
        fills = also.get(f"T{T0}_{S0}slots_with_fills", {})
        pol = HEAD_POLICY if HEAD_POLICY in fills else next(iter(fills), None)
        if pol is not None:
            head = fills[pol]
            head_desc = (f"through the workload's own cache of {S0} slots ({cfg['residency']} "
                         f"initial residency), misses filled from pinned host memory over PCIe "
                         f"on the side stream, {POLICY_DESC.get(pol, pol)}")
    ffn = hit["ffn"]
    line = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "int4g128": "int4 weights x int8 activations"}[shape.wfmt],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: E={shape.E} top-{shape.k}, H={shape.H}, F={shape.F}"
                               + (f", {shape.n_shared} shared" if shape.n_shared else "")
                               + (f", {shape.layers} layers" if shape.layers > 1 else "")
                               + f", decode {head['tokens_per_step']} token/step " + head_desc,
                   "tokens_per_step": head["tokens_per_step"], "hit_rate": head.get("hit_rate"),
                   "fills_per_step": head.get("fills_per_step"),
                   # the fills' bytes over the whole step time, against one copy's rate alone
                   "fill_gbs_in_step": (round(head["fill_bytes_per_step"] / head["ms_per_step"] / 1e6, 2)
                                        if head.get("fill_bytes_per_step") else None),
                   "pcie_copy_gbs": also.get("pcie_copy", {}).get("gbs"),
                   "pool_replicas": head["pool_replicas"], "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "moe_expert_ffn, one call per layer step (at one token one launch of "
                               "both passes, the work list written by the router's select), "
                               f"{hit_T} token/step, all routed experts resident",
                     "bound": "hbm", "achieved": round(ffn["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ffn["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"{args.workload}/decode{hit_T}",
                                                 f"{args.workload}/T{hit_T}"),
                     "avg_us": round(ffn["avg_us"], 2), "bytes_per_call": int(ffn["bytes_per_call"])},
        "also": also,
    }
    if not args.no_cpu_baseline and shape.layers == 1:
        line["cpu_baseline"] = cpu_baseline(shape)
        line["cpu_baseline"]["tiny_fp32_one_thread"] = cpu_baseline_tiny()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
