"""End-to-end parity of each workload at its own full shape and its own cache.

Every step runs through the layer runtime (route, permute, residency plan,
fills from the pinned host store in waves, expert FFN over the slots, shared
experts, combine) and is compared with the oracle's layer over its own slot pool
(tests/gpu_common.run_layer_case): routing stage parity, bit-exact permutation
and slot tables after every step, and the output within the format's tolerance
over every token (DeepSeek-V3-shaped prefill of 4096 tokens: a fixed sample of
tokens, computed one by one by the oracle).
"""
import numpy as np
import pytest
import torch

import oracle as O
from expert_offload_routed_amd import workloads as W
from gpu_common import OracleWeights, run_layer_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _cfg(name):
    cfg = W.WORKLOADS[name]
    return cfg["shape"], cfg


@pytest.mark.timeout(900)
def test_mixtral_prefill512_on_its_4_of_8_cache():
    """512 tokens route to all 8 experts with 4 slots: fills in waves (some slots refilled
    after their expert was computed), then a decode step on the resulting cache."""
    shape, cfg = _cfg("mixtral_e8k2_h4096_f14336_bf16")
    run_layer_case(shape, cfg["slots"][0], cfg["residency"], [512, 1])


@pytest.mark.timeout(900)
def test_qwen3_stack_48_layers_shared_pool():
    """All 48 layers x 128 experts over one pool of 2765 slots (45% of the layer-experts),
    decode 1 then 16 tokens: every layer's routing, tables and output at every step."""
    shape, cfg = _cfg("qwen3moe_l48_e128k8_h2048_f768_bf16")
    run_layer_case(shape, cfg["slots"][0], cfg["residency"], [1, 16],
                   layers_order=list(range(shape.layers)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("slots", [16, 32, 48])
def test_dsv2lite_caches(slots):
    """64 routed experts (top-6) plus 2 shared, at 25/50/75% cached, through decode and
    the prefill sizes 32, 256 and 1024 (several waves once the routed set exceeds the
    slots)."""
    shape, cfg = _cfg("dsv2lite_e64k6s2_h2048_f1408_bf16")
    run_layer_case(shape, slots, cfg["residency"], [1, 32, 256, 1024])


def _sampler(n_tokens, max_experts, seed=0):
    """A fixed sample of tokens for the oracle to compute one by one: the first and the
    last token, then tokens in a seeded order while the experts they route to stay within
    max_experts (each expert the oracle computes costs a dequantisation)."""
    def pick(T, ids):
        if T <= 64:
            return None
        order = [0, T - 1] + np.random.default_rng(seed).permutation(np.arange(1, T - 1)).tolist()
        rows, experts = [], set()
        for t in order:
            new = experts | {int(e) for e in ids[t]}
            if len(new) <= max_experts:
                rows.append(t)
                experts = new
            if len(rows) == n_tokens:
                break
        say(f"  sampled {len(rows)} tokens over {len(experts)} experts")
        return sorted(rows)
    return pick


@pytest.mark.timeout(900)
def test_dsv3_int4_84_slots():
    """256 int4 experts (top-8) plus one shared, 84 slots: decode 1 and 32 tokens (every
    token), prefill 4096 (every routed expert, misses in waves; sampled tokens), and a
    decode step after it."""
    shape, cfg = _cfg("dsv3_e256k8s1_h7168_f2048_int4")
    run_layer_case(shape, cfg["slots"][0], cfg["residency"], [1, 32, 4096, 1],
                   sample=_sampler(24, 48))
