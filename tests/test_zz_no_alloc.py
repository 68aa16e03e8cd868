"""moe_expert_ffn_noalloc (workspace in a static device array) against moe_expert_ffn.

Two calls in a row on the same GPU, the second with a smaller input, each compared
bit for bit with moe_expert_ffn on the same inputs (same kernels, so the same bits;
the oracle bar is then met by the tests of moe_expert_ffn). Sizes beyond the array
are rejected."""
import numpy as np
import pytest
import torch

from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import harness as Hn
from expert_offload_routed_amd import workloads as W
from gpu_common import say

pytestmark = pytest.mark.gpu


def _case(shape, T, seed):
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    store = Hn.ExpertStore(shape)
    perm_slots = np.random.default_rng(seed).permutation(E)
    pool = torch.empty(E * store.stride, dtype=torch.uint8, device="cuda")
    for e in range(E):
        s = int(perm_slots[e])
        pool[s * store.stride:(s + 1) * store.stride].copy_(store.host[W.blob_of(shape, 0, e)])
    lut = torch.from_numpy(perm_slots.astype(np.int32)).to("cuda")
    x = W.tokens(shape, T, step=seed, device="cuda")
    wr, b = W.router(shape, device="cuda")
    _, ids, _ = B.moe_route(x, wr, b, k)
    p = B.moe_permute(ids, E)
    return x, p, lut, pool, store.stride


@pytest.mark.parametrize("shape,Ts", [
    (W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), E=12, k=8, H=7168, F=2048), (24, 1)),
    (W.reduced(W.shape_of("mixtral_e8k2_h4096_f14336_bf16"), E=16, k=4, H=512, F=384), (300, 40)),
])
def test_noalloc_matches_workspace_entry(shape, Ts):
    wcode = Hn.WFMT_CODE[shape.wfmt]
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    for i, T in enumerate(Ts):  # two calls in a row, the second smaller
        say(f"noalloc {shape.name} T={T}")
        x, p, lut, pool, stride = _case(shape, T, 10 + i)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y_ref = torch.zeros(T * k, H, dtype=torch.float32, device="cuda")
        ws = torch.zeros(B.moe_ffn_workspace_bytes(T, H, F, E, k, wcode), dtype=torch.uint8, device="cuda")
        B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, wcode, T, H, F, E, k,
                         y_ref, err, ws)
        y = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_expert_ffn_noalloc(x, p["perm"], p["offsets"], lut, None, pool, stride, wcode, T, H, F,
                                 E, k, y, err)
        torch.cuda.synchronize()
        assert err.item() == 0
        assert torch.equal(y, y_ref), (T, float((y - y_ref).abs().max()))


def test_noalloc_rejects_sizes_beyond_its_array():
    shape = W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), E=12, k=8, H=7168, F=2048)
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    T = 4096  # the workspace of 4096 tokens x 8 experts exceeds the array
    assert B.moe_ffn_workspace_bytes(T, H, F, E, k, B.MOE_INT4G128) > B.moe_noalloc_scratch_bytes()
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    perm = torch.zeros(T * k, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    lut = torch.zeros(E, dtype=torch.int32, device="cuda")
    pool = torch.zeros(B.moe_slot_layout(H, F, B.MOE_INT4G128)["slot_bytes"], dtype=torch.uint8,
                       device="cuda")
    y = torch.zeros(T * k, H, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoeError):
        B.moe_expert_ffn_noalloc(x, perm, offsets, lut, None, pool, pool.numel(), B.MOE_INT4G128, T, H,
                                 F, E, k, y, err)
