"""GPU parity of every C-ABI stage against the oracle, then the whole layer.

Bars: integer outputs (ids, counts, offsets, perm, inv, distinct, tables) are
bit-exact; routing weights within 1e-6 absolute; expert outputs and the layer
output within 1e-5 relative L2 (fp32) or 2e-2 (bf16 / int4).
"""
import numpy as np
import pytest
import torch

import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import harness as Hn
from expert_offload_routed_amd import workloads as W
from gpu_common import (TOL, OracleWeights, check_routing, oracle_y_rows, rel_l2,
                        run_layer_case as _run_layer_case, say)

pytestmark = pytest.mark.gpu

TINY = W.shape_of("tiny_e8k2_h256_f512_fp32")
MIX = W.shape_of("mixtral_e8k2_h4096_f14336_bf16")
DSV3 = W.shape_of("dsv3_e256k8s1_h7168_f2048_int4")


def _dev():
    return torch.device("cuda:0")


# ------------------------------------------------------------------ routing --
ROUTE_CASES = [
    (TINY, 16), (TINY, 1),
    (W.reduced(MIX, E=8, k=2, H=4096), 37),
    (W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), H=2048), 300),
    (W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), H=7168), 64),
    (W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), H=7168), 4096),  # prefill size
    (W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), E=96, k=6, H=1024), 1000),  # ragged tiles
    (W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), E=40, k=4, H=520), 100),  # H not a multiple
                                                                                      # of 64: FMA logits
    (W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), E=1000, k=16, H=512), 9),
    (W.reduced(TINY, E=5, k=5, H=24), 3),
]


@pytest.mark.parametrize("shape,T", ROUTE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_route_stage(shape, T):
    say(f"route {shape.name} T={T}")
    x = W.tokens(shape, T, device=_dev())
    wr, b = W.router(shape, device=_dev())
    logits, ids, w = B.moe_route(x, wr, b, shape.k)
    torch.cuda.synchronize()
    under, err = check_routing(x, wr, b, shape.k, logits, ids, w)
    say(f"  max logit err {err:.2e}, tokens under margin {under}")
    assert np.all(np.abs(w.sum(1).cpu().numpy() - 1.0) <= 1e-6)


def test_route_renorm_off_and_no_bias():
    shape = W.reduced(TINY, E=16, k=3, H=64)
    x = W.tokens(shape, 10, device=_dev())
    wr, _ = W.router(shape, device=_dev())
    logits, ids, w = B.moe_route(x, wr, None, 3, renorm=False)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    np.testing.assert_allclose(lg, O.router_logits(x, wr, None), rtol=0, atol=1e-5)
    ig = ids.cpu().numpy()
    assert np.array_equal(O.select_topk(lg, 3), ig)
    np.testing.assert_allclose(w.cpu().numpy(), O.gate_weights(lg.astype(np.float64), ig, renorm=False),
                               atol=1e-6)


def test_route_empty_is_noop():
    shape = TINY
    x = torch.empty(0, shape.H, device=_dev())
    wr, b = W.router(shape, device=_dev())
    logits, ids, w = B.moe_route(x, wr, b, 2)
    torch.cuda.synchronize()
    assert ids.numel() == 0


def test_route_rejects_bad_args():
    x = W.tokens(TINY, 4, device=_dev())
    wr, b = W.router(TINY, device=_dev())
    with pytest.raises(B.MoeError):
        B.moe_route(x, wr, b, 9)  # k > E
    with pytest.raises(B.MoeError):
        B.moe_route(x[:, :250].contiguous(), wr[:, :250].contiguous(), b, 2)  # H % 8 != 0


@pytest.mark.parametrize("shape,T", [(TINY, 16), (TINY, 1), (W.reduced(MIX, H=4096), 5),
                                     (W.reduced(DSV3, H=7168), 16), (W.reduced(DSV3, H=512), 40),
                                     (W.reduced(TINY, E=64, k=64, H=64), 16),
                                     (W.reduced(TINY, E=5, k=3, H=264), 7),     # one workgroup, 3 H slices per expert
                                     (W.reduced(MIX, E=40, k=4, H=1024), 11),   # one workgroup, 40 (expert, slice) pairs
                                     (W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), H=2048), 3),
                                     (W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), E=1000, k=16, H=512), 9),
                                     # one token: logits, then the one-wave select (k <= 64)
                                     (W.reduced(DSV3, H=7168), 1),
                                     (W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), 1),
                                     (W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), E=1000, k=16, H=512), 1),
                                     (W.reduced(TINY, E=64, k=64, H=64), 1),
                                     (W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), H=2048), 1)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_route_permute_fused(shape, T):
    """One-launch front end (T <= 16), the one-token select, and the two-call fallback: same bar
    as the separate stages."""
    say(f"route_permute {shape.name} T={T}")
    counter = torch.zeros(1, dtype=torch.int32, device=_dev())
    for rep in range(3):  # the counter must come back to zero after every call
        x = W.tokens(shape, T, step=rep, device=_dev())
        wr, b = W.router(shape, device=_dev())
        logits, ids, w, p = B.moe_route_permute(x, wr, b, shape.k, sync_counter=counter)
        torch.cuda.synchronize()
        assert counter.item() == 0
        check_routing(x, wr, b, shape.k, logits, ids, w)
        ref = O.permute(ids.cpu().numpy(), shape.E)
        n = T * shape.k
        assert p["counts"].cpu().numpy().tolist() == ref["counts"].tolist()
        assert p["offsets"].cpu().numpy().tolist() == ref["offsets"].tolist()
        assert p["perm"].cpu().numpy()[:n].tolist() == ref["perm"].tolist()
        assert p["inv"].cpu().numpy()[:n].tolist() == ref["inv"].tolist()
        nd = int(p["n_distinct"].item())
        assert p["distinct"].cpu().numpy()[:nd].tolist() == ref["distinct"].tolist()


# -------------------------------------------------------------- permutation --
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (513, 64, 6), (4096, 256, 8),
                                   (77, 1024, 16), (3, 1, 1),
                                   (9001, 64, 6),    # 54006 picks: two rounds of the rank kernel
                                   (20000, 8, 2)])   # 40000 picks, one expert in almost every row
def test_permute_stage(T, E, k):
    say(f"permute T={T} E={E} k={k}")
    g = torch.Generator().manual_seed(T * 7 + E)
    # distinct ids per row, Zipf-like skew through sorting random keys with a bias
    keys = torch.rand(T, E, generator=g) + torch.linspace(0, 2, E)
    ids = torch.argsort(keys, dim=1)[:, :k].to(torch.int32)
    out = B.moe_permute(ids.to(_dev()), E)
    torch.cuda.synchronize()
    ref = O.permute(ids.numpy(), E)
    assert out["counts"].cpu().numpy().tolist() == ref["counts"].tolist()
    assert out["offsets"].cpu().numpy().tolist() == ref["offsets"].tolist()
    assert out["perm"].cpu().numpy()[:T * k].tolist() == ref["perm"].tolist()
    assert out["inv"].cpu().numpy()[:T * k].tolist() == ref["inv"].tolist()
    nd = int(out["n_distinct"].item())
    assert out["distinct"].cpu().numpy()[:nd].tolist() == ref["distinct"].tolist()


def test_permute_empty():
    out = B.moe_permute(torch.empty(0, 2, dtype=torch.int32, device=_dev()), 8)
    torch.cuda.synchronize()
    assert out["counts"].sum().item() == 0 and out["n_distinct"].item() == 0
    assert out["offsets"].cpu().tolist() == [0] * 9


# --------------------------------------------------------------- expert FFN --
def _pool_with(shape, lut_perm, layer=0):
    """Pool of E slots holding expert e in slot lut_perm[e] (packed on the host, copied)."""
    store = Hn.ExpertStore(shape)
    E = shape.E
    pool = torch.empty(E * store.stride, dtype=torch.uint8, device=_dev())
    for e in range(E):
        s = lut_perm[e]
        pool[s * store.stride:(s + 1) * store.stride].copy_(store.host[W.blob_of(shape, layer, e)])
    return pool, store.stride, torch.tensor(lut_perm, dtype=torch.int32, device=_dev())


FFN_CASES = [
    (TINY, 16),
    (W.reduced(MIX, E=16, k=4, H=512, F=384), 1),
    (W.reduced(MIX, E=16, k=4, H=512, F=384), 3),
    (W.reduced(MIX, E=16, k=4, H=512, F=384), 40),    # GEMV groups and MFMA tiles
    (W.reduced(MIX, E=16, k=4, H=512, F=384), 300),   # several 64-row tiles, ragged tails
    (W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), E=16, k=6, H=2048, F=1408), 100),
    # one token, bf16: both passes over even shares of row blocks in one launch
    (W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), E=16, k=6, H=2048, F=1408), 1),
    (W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), E=16, k=8, H=2048, F=768), 1),
    (W.reduced(MIX, E=4, k=4, H=4096, F=14336), 1),    # shares of 14 row blocks
    (W.reduced(MIX, E=8, k=2, H=256, F=512, wfmt="f32", xfmt="f32"), 29),
    (W.reduced(DSV3, E=16, k=4, H=512, F=256), 1),     # int4 weights, int8 activations
    (W.reduced(DSV3, E=16, k=4, H=512, F=256), 3),
    (W.reduced(DSV3, E=16, k=4, H=512, F=256), 40),
    (W.reduced(DSV3, E=16, k=4, H=512, F=256), 300),
    (W.reduced(DSV3, E=12, k=8, H=7168, F=2048), 1),  # full sizes, one token: workgroups take
                                                       # several units of the gate/up pass
    (W.reduced(DSV3, E=12, k=8, H=7168, F=2048), 2),  # full hidden/FFN sizes
    (W.reduced(DSV3, E=12, k=8, H=7168, F=2048), 24),
    (W.reduced(DSV3, E=12, k=8, H=7168, F=2048), 200),  # every group on MFMA tiles, some > 128 rows
    (W.reduced(DSV3, E=8, k=4, H=384, F=384), 40),     # 3 scale groups per row, partial 256-row tiles
    (W.reduced(DSV3, E=8, k=4, H=384, F=384), 300),
]


@pytest.mark.parametrize("shape,T", FFN_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_expert_ffn_stage(shape, T):
    say(f"ffn {shape.name} T={T}")
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    rng = np.random.default_rng(T)
    lut_perm = rng.permutation(E).tolist()
    pool, stride, lut = _pool_with(shape, lut_perm)
    x = W.tokens(shape, T, device=_dev())
    wr, b = W.router(shape, device=_dev())
    _, ids, _ = B.moe_route(x, wr, b, k)
    p = B.moe_permute(ids, E)
    wcode = Hn.WFMT_CODE[shape.wfmt]
    ws = torch.empty(B.moe_ffn_workspace_bytes(T, H, F, E, k, wcode), dtype=torch.uint8, device=_dev())
    y = torch.zeros(T * k, H, dtype=torch.float32, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, wcode, T, H, F, E, k, y, err, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    ids_np = ids.cpu().numpy()
    ref = O.permute(ids_np, E)
    yr = oracle_y_rows(shape, x, ids_np, ref["perm"], ref["offsets"], 0, ref["distinct"])
    r = rel_l2(y.cpu().numpy(), yr)
    say(f"  rel L2 {r:.3e}")
    assert r <= TOL[shape.wfmt]
    # relabelled slots give bitwise the same rows
    pool2, _, lut2 = _pool_with(shape, list(range(E)))
    y2 = torch.zeros_like(y)
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut2, None, pool2, stride, wcode, T, H, F, E, k, y2, err, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # determinism
    y3 = torch.zeros_like(y)
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, wcode, T, H, F, E, k, y3, err, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y3)


def test_expert_ffn_absent_expert_sets_error_and_skips():
    shape = W.reduced(MIX, E=8, k=2, H=256, F=256)
    E, k, H, F, T = 8, 2, 256, 256, 12
    pool, stride, lut = _pool_with(shape, list(range(E)))
    x = W.tokens(shape, T, device=_dev())
    wr, b = W.router(shape, device=_dev())
    _, ids, _ = B.moe_route(x, wr, b, k)
    p = B.moe_permute(ids, E)
    torch.cuda.synchronize()
    e_missing = int(ids[0, 0].item())
    lut[e_missing] = -1
    ws = torch.empty(B.moe_ffn_workspace_bytes(T, H, F, E, k, 1), dtype=torch.uint8, device=_dev())
    y = torch.full((T * k, H), 7.0, dtype=torch.float32, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, 1, T, H, F, E, k, y, err, ws)
    torch.cuda.synchronize()
    assert err.item() & B.MOE_ERR_ABSENT
    o = p["offsets"].cpu().numpy()
    assert torch.all(y[o[e_missing]:o[e_missing + 1]] == 7.0)
    other = [r for r in range(T * k) if not (o[e_missing] <= r < o[e_missing + 1])]
    assert torch.all(y[other] != 7.0)


def test_expert_ffn_and_combine_empty_calls():
    """No tokens: the FFN stage (bf16 and int4 slots) and the combine succeed, leave the error
    word at zero and write nothing; an output that lives inside a sentinel buffer stays intact."""
    for shape in (W.reduced(MIX, E=8, k=2, H=256, F=256), W.reduced(DSV3, E=16, k=4, H=512, F=256)):
        say(f"empty calls {shape.name}")
        E, k, H, F = shape.E, shape.k, shape.H, shape.F
        pool, stride, lut = _pool_with(shape, list(range(E)))
        wcode = Hn.WFMT_CODE[shape.wfmt]
        x = torch.empty(0, H, dtype=torch.bfloat16, device=_dev())
        perm = torch.empty(0, dtype=torch.int32, device=_dev())
        offsets = torch.zeros(E + 1, dtype=torch.int32, device=_dev())
        ws = torch.empty(B.moe_ffn_workspace_bytes(0, H, F, E, k, wcode), dtype=torch.uint8, device=_dev())
        big = torch.full((4, H), 7.0, dtype=torch.float32, device=_dev())
        err = torch.zeros(1, dtype=torch.int32, device=_dev())
        B.moe_expert_ffn(x, perm, offsets, lut, None, pool, stride, wcode, 0, H, F, E, k, big[:0], err, ws)
        inv = torch.empty(0, dtype=torch.int32, device=_dev())
        w = torch.empty(0, k, dtype=torch.float32, device=_dev())
        out = B.moe_combine(big[:0], inv, w, 0, k, H, None, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert err.item() == 0
        assert out.shape == (0, H)
        assert torch.all(big == 7.0)


# ------------------------------------------------------------------ combine --
@pytest.mark.parametrize("T,k,H,n_sh,out", [(16, 2, 256, 0, torch.float32), (33, 6, 2048, 2, torch.bfloat16),
                                            (1, 8, 7168, 1, torch.bfloat16), (1, 2, 256, 0, torch.float32),
                                            (1, 6, 2048, 2, torch.float32),
                                            (5, 12, 512, 1, torch.float32)])  # two row batches
def test_combine_stage(T, k, H, n_sh, out):
    g = torch.Generator().manual_seed(T + k)
    E = 4 * k
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    pr = O.permute(ids.numpy(), E)
    y = torch.randn(T * k, H, generator=g)
    w = torch.rand(T, k, generator=g)
    w[0, -1] = 0.0
    y[pr["inv"][k - 1]] = float("nan")  # the zero-weight row of token 0 is poisoned
    sh = torch.randn(n_sh, T, H, generator=g) if n_sh else None
    res = B.moe_combine(y.to(_dev()), torch.from_numpy(pr["inv"]).to(_dev()), w.to(_dev()), T, k, H,
                        None if sh is None else sh.to(_dev()), out_dtype=out)
    torch.cuda.synchronize()
    y_assign = y.numpy()[pr["inv"]].reshape(T, k, H)
    ref = O.combine(y_assign, w.numpy(), None if sh is None else sh.numpy())
    got = res.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    tol = 1e-6 if out == torch.float32 else 8e-3
    assert rel_l2(got, ref) <= tol


# ---------------------------------------------------------------- slot fill --
def test_slot_fill_and_tag_commit():
    shape = W.reduced(MIX, E=6, k=2, H=256, F=128)
    store = Hn.ExpertStore(shape)
    S, E = 3, 6
    pool = torch.zeros(S * store.stride, dtype=torch.uint8, device=_dev())
    lut = torch.full((2 * E,), -1, dtype=torch.int32, device=_dev())
    owner = torch.full((S,), -1, dtype=torch.int32, device=_dev())
    tags = torch.zeros(S, dtype=torch.int64, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    fs = torch.cuda.Stream()
    cs = torch.cuda.current_stream()
    B.slot_fill(pool, store.stride, 1, store.host[4], store.stride, lut, E + 4, owner, tags, 5, err, fs, cs)
    torch.cuda.synchronize()
    assert torch.equal(pool[store.stride:2 * store.stride].cpu(), store.host[4])
    assert lut.cpu().tolist() == [-1] * (E + 4) + [1, -1]
    assert owner.cpu().tolist() == [-1, E + 4, -1] and tags.cpu().tolist() == [0, 5, 0]
    # replacing the owner of slot 1 clears the old table entry
    B.slot_fill(pool, store.stride, 1, store.host[2], store.stride, lut, 2, owner, tags, 6, err, fs, cs)
    torch.cuda.synchronize()
    assert lut.cpu().tolist()[2] == 1 and lut.cpu().tolist()[E + 4] == -1 and err.item() == 0
    # a commit whose tag was superseded is refused and leaves the tables alone
    tags[0] = 9
    torch.cuda.synchronize()
    B.slot_commit(lut, 3, owner, 0, tags, 8, err)
    torch.cuda.synchronize()
    assert err.item() == B.MOE_ERR_STALE_TAG
    assert lut.cpu().tolist()[3] == -1 and owner.cpu().tolist()[0] == -1


def test_slot_fill_copy_kernel_and_transfer_paths():
    """A fill copies with a kernel when the pinned source and the sizes are 16-byte aligned,
    else with a copy-engine transfer: both land the same bytes."""
    shape = W.reduced(MIX, E=6, k=2, H=256, F=128)
    store = Hn.ExpertStore(shape)
    S, E = 2, 6
    pool = torch.zeros(S * store.stride, dtype=torch.uint8, device=_dev())
    lut = torch.full((E,), -1, dtype=torch.int32, device=_dev())
    owner = torch.full((S,), -1, dtype=torch.int32, device=_dev())
    tags = torch.zeros(S, dtype=torch.int64, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    base = store.host[3].data_ptr()
    # aligned interior source, 4096 bytes: the copy kernel
    B.slot_fill(pool, store.stride, 0, base + 256, 4096, lut, 1, owner, tags, 3, err)
    # source 8 bytes past alignment, 1000 bytes: the transfer
    B.slot_fill(pool, store.stride, 1, base + 8, 1000, lut, 2, owner, tags, 4, err)
    torch.cuda.synchronize()
    flat = store.host[3]
    assert torch.equal(pool[:4096].cpu(), flat[256:256 + 4096])
    assert torch.equal(pool[store.stride:store.stride + 1000].cpu(), flat[8:1008])
    assert err.item() == 0 and owner.cpu().tolist() == [1, 2]


def test_slot_fill_rejects_pageable_host_memory():
    pool = torch.zeros(8192, dtype=torch.uint8, device=_dev())
    lut = torch.full((4,), -1, dtype=torch.int32, device=_dev())
    owner = torch.full((2,), -1, dtype=torch.int32, device=_dev())
    tags = torch.zeros(2, dtype=torch.int64, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    pageable = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(B.MoeError):
        B.slot_fill(pool, 4096, 0, pageable, 4096, lut, 0, owner, tags, 1, err)


# --------------------------------------------------------------- whole layer --
def test_layer_tiny_fp32_identity():
    _run_layer_case(TINY, 8, "identity", [16, 16])


def test_layer_bf16_misses_multiwave():
    shape = W.reduced(MIX, E=12, k=3, H=256, F=256)
    _run_layer_case(shape, 5, "random", [1, 8, 40, 2, 40])


def test_layer_stack_shared_pool():
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    _run_layer_case(shape, 14, "zipf_rank", [1, 3, 16], layers_order=[0, 1, 2])


def test_layer_stack_policy_mrs():
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    _run_layer_case(shape, 14, "zipf_rank", [1, 3, 1, 16, 2, 1], layers_order=[0, 1, 2],
                    policy=(B.MOE_POLICY_MRS, 4, None))


def test_layer_policy_history_shared_experts():
    shape = W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), E=16, k=6, H=256, F=256)
    _run_layer_case(shape, 8, "zipf_rank", [1, 2, 32, 1, 5, 3],
                    policy=(B.MOE_POLICY_HISTORY, 6, [1.0, 0.5, 2.0, 0.25, 0.8]))


def test_layer_stack_device_orchestration():
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    _run_layer_case(shape, 14, "zipf_rank", [1, 3, 1, 2, 1, 3], layers_order=[0, 1, 2], device_plan=True)


def test_layer_stack_device_orchestration_mrs():
    """Minus Recent Score planned on the device: routing, tables and outputs those of the
    oracle's scored planner at every layer-step of a 3-layer stack."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    _run_layer_case(shape, 14, "zipf_rank", [1, 3, 1, 2, 1, 3, 1], layers_order=[0, 1, 2],
                    device_plan=True, policy=(B.MOE_POLICY_MRS, 4, None))


def test_layer_device_orchestration_mrs_shared_experts_int4():
    shape = W.reduced(DSV3, E=32, k=8, H=256, F=128)
    _run_layer_case(shape, 12, "zipf_rank", [1, 1, 1, 1, 1, 1, 1, 1], device_plan=True,
                    policy=(B.MOE_POLICY_MRS, 8, None))


HIST_PARAMS = [1.0, 0.5, 2.0, 0.25, 0.8]


def test_layer_stack_device_orchestration_history():
    """The routing-history score planned on the device: routing, tables and outputs those of
    the oracle's scored planner at every layer-step of a 3-layer stack."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    _run_layer_case(shape, 14, "zipf_rank", [1, 3, 1, 2, 1, 3, 1, 2], layers_order=[0, 1, 2],
                    device_plan=True, policy=(B.MOE_POLICY_HISTORY, 4, HIST_PARAMS))


def test_layer_device_orchestration_history_shared_experts_int4():
    shape = W.reduced(DSV3, E=32, k=8, H=256, F=128)
    _run_layer_case(shape, 12, "zipf_rank", [1, 1, 1, 1, 1, 1, 1, 1], device_plan=True,
                    policy=(B.MOE_POLICY_HISTORY, 3, [0.0, 1.0, 0.5, 1.0, 0.5]))


@pytest.mark.parametrize("kind", ["mrs", "history"])
def test_device_orchestration_hands_mrs_history_back_and_forth(kind):
    """Host plans under an eviction score, then the device, then the host again: one history
    and one set of tables, those of the oracle's scored planner."""
    shape = W.reduced(MIX, E=12, k=3, H=256, F=256)
    slots, window = 5, 3
    residency = W.initial_residency(shape, slots, "random")
    layer_obj = Hn.SlotCacheLayer(shape, slots, residency, 4)
    if kind == "mrs":
        layer_obj.ctx.set_policy(B.MOE_POLICY_MRS, window, None)
        pol = O.MinusRecentScore(1, shape.E, window)
    else:
        layer_obj.ctx.set_policy(B.MOE_POLICY_HISTORY, window, HIST_PARAMS)
        pol = O.RoutingHistoryScore(1, shape.E, window, weights=HIST_PARAMS[:4], lam=HIST_PARAMS[4])
    planner = O.ScoredSlotPlanner(slots, 1, shape.E, pol, residency)
    for step in range(8):
        layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE if step in (2, 3, 4) else B.MOE_ORCH_HOST)
        say(f"{kind} handoff step={step}")
        x = W.tokens(shape, 1, step=step, device=_dev())
        layer_obj.forward(x)
        torch.cuda.synchronize()
        assert layer_obj.err.item() == 0
        sc = layer_obj.ctx.step_scores()
        ids = layer_obj.outputs(1)["ids"].cpu().numpy()
        planner.plan(0, O.permute(ids, shape.E)["distinct"], sc)
        lut_h, _, last_use_h, clock_h = layer_obj.tables()
        assert lut_h.tolist() == planner.lut[0].tolist()
        assert last_use_h.tolist() == planner.last_use and clock_h == planner.clock


def test_layer_device_orchestration_shared_experts_int4():
    shape = W.reduced(DSV3, E=32, k=8, H=256, F=128)
    _run_layer_case(shape, 12, "zipf_rank", [1, 1, 1, 1], device_plan=True)


def test_device_orchestration_hands_tables_back_and_forth():
    """Host plans, then device plans, then host again: the tables follow one LRU history."""
    shape = W.reduced(MIX, E=12, k=3, H=256, F=256)
    slots = 5
    residency = W.initial_residency(shape, slots, "random")
    layer_obj = Hn.SlotCacheLayer(shape, slots, residency, 4)
    planner = O.LruSlotPlanner(slots, 1, shape.E, residency)
    n_distinct = n_fills = 0
    for step, T in enumerate([1, 1, 1, 1, 1, 1]):
        layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE if step in (2, 3) else B.MOE_ORCH_HOST)
        say(f"handoff step={step}")
        x = W.tokens(shape, T, step=step, device=_dev())
        layer_obj.forward(x)
        torch.cuda.synchronize()
        ids = layer_obj.outputs(T)["ids"].cpu().numpy()
        distinct = O.permute(ids, shape.E)["distinct"]
        waves = planner.plan(0, distinct)
        n_distinct += len(distinct)
        n_fills += sum(len(w.fills) for w in waves)
        lut_h, _, last_use_h, clock_h = layer_obj.tables()
        assert lut_h.tolist() == planner.lut[0].tolist()
        assert last_use_h.tolist() == planner.last_use and clock_h == planner.clock
    cnt = layer_obj.counters()
    assert cnt["distinct"] == n_distinct and cnt["fills"] == n_fills


@pytest.mark.parametrize("layers,policy", [(3, "lru"), (1, "lru"), (3, "mrs"), (1, "history")])
def test_device_orchestrated_stack_step_replays_as_a_graph(layers, policy):
    """A whole stack step (every layer) planned and filled on the device is captured once and
    replayed; between replays the inputs change in place (so replays miss and fill). Every
    replay equals an eager device-orchestrated context fed the same inputs (a 3-layer stack,
    and one layer whose random initial residency makes most steps fill), under LRU and under
    both eviction scores (their history recorded on the device by the captured kernels)."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=layers, E=16, k=4,
                      H=256, F=128, blobs=16)
    L, T = shape.layers, 1
    slots = 14 if L > 1 else 5
    residency = W.initial_residency(shape, slots, "zipf_rank" if L > 1 else "random")
    s = torch.cuda.Stream()
    graphed = Hn.SlotCacheLayer(shape, slots, residency, T, compute_stream=s)
    eager = Hn.SlotCacheLayer(shape, slots, residency, T, store=graphed.store)
    for lay in (graphed, eager):
        if policy == "mrs":
            lay.ctx.set_policy(B.MOE_POLICY_MRS, 3, None)
        elif policy == "history":
            lay.ctx.set_policy(B.MOE_POLICY_HISTORY, 3, HIST_PARAMS)
        lay.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    xs = [W.tokens(shape, T, layer=l, step=0, device=_dev()) for l in range(L)]
    outs_g = [torch.empty(T, shape.H, dtype=graphed.out_dtype, device=_dev()) for _ in range(L)]
    outs_e = [torch.empty_like(o) for o in outs_g]

    def stack_step(lay, outs):
        for l in range(L):
            lay.forward(xs[l], layer=l, out=outs[l])

    with torch.cuda.stream(s):
        stack_step(graphed, outs_g)  # eager first step (per-T set-up stays out of the graph)
    stack_step(eager, outs_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        stack_step(graphed, outs_g)
    torch.cuda.synchronize()  # the capture ran nothing: both contexts have done step 0 once
    for rep in range(5):
        say(f"graph replay {rep}")
        for l in range(L):  # eager work between replays: new inputs, in place
            xs[l].copy_(W.tokens(shape, T, layer=l, step=rep + 1, device=_dev()))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        stack_step(eager, outs_e)
        torch.cuda.synchronize()
        assert graphed.err.item() == 0 and eager.err.item() == 0
        for l in range(L):
            assert torch.equal(outs_g[l], outs_e[l]), (rep, l)
        tg, te = graphed.tables(), eager.tables()
        assert tg[0].tolist() == te[0].tolist() and tg[2].tolist() == te[2].tolist() and tg[3] == te[3]
    cg, ce = graphed.counters(), eager.counters()
    assert cg == ce and cg["fills"] > 0


def test_device_orchestration_rejects_more_routed_than_slots():
    shape = W.reduced(MIX, E=12, k=3, H=256, F=256)
    layer_obj = Hn.SlotCacheLayer(shape, 4, W.initial_residency(shape, 4, "random"), 8)
    layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    x = W.tokens(shape, 2, step=0, device=_dev())  # T*k = 6 > 4 slots
    with pytest.raises(B.MoeError):
        layer_obj.forward(x)


@pytest.mark.parametrize("kind", ["mrs", "history"])
def test_device_orchestration_policy_window_limit(kind):
    """The device planner keeps an eviction-score history of at most 16 steps: a longer
    window is refused (invalid argument) whichever of the two settings comes second, and the
    context keeps planning under its previous setting."""
    shape = W.reduced(MIX, E=12, k=3, H=256, F=256)
    pol = B.MOE_POLICY_MRS if kind == "mrs" else B.MOE_POLICY_HISTORY
    params = None if kind == "mrs" else HIST_PARAMS
    layer_obj = Hn.SlotCacheLayer(shape, 5, W.initial_residency(shape, 5, "random"), 4)
    layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    with pytest.raises(B.MoeError) as e:
        layer_obj.ctx.set_policy(pol, 17, params)
    assert e.value.rc == -1
    layer_obj.ctx.set_policy(pol, 16, params)  # the largest window the device keeps
    layer_obj.forward(W.tokens(shape, 1, step=0, device=_dev()))
    torch.cuda.synchronize()
    assert layer_obj.err.item() == 0
    layer_obj.ctx.set_orchestration(B.MOE_ORCH_HOST)
    layer_obj.ctx.set_policy(pol, 17, params)  # the host keeps any window
    with pytest.raises(B.MoeError) as e:
        layer_obj.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    assert e.value.rc == -1
    layer_obj.forward(W.tokens(shape, 1, step=1, device=_dev()))  # still planned on the host
    torch.cuda.synchronize()
    assert layer_obj.err.item() == 0


SPLIT = W.reduced(DSV3, wfmt="int4g128_resplit")


def test_layer_split_precision_misses_shared():
    """Split-precision experts with misses (fills in waves) and a shared expert (always W^H)."""
    shape = W.reduced(SPLIT, E=16, k=4, H=256, F=128, layers=2)
    _run_layer_case(shape, 12, "zipf_rank", [1, 4, 2, 24, 1], layers_order=[0, 1],
                    split=(0.125, [1.0, 0.5], 0.75))


def test_layer_split_precision_all_resident():
    shape = W.reduced(SPLIT, E=16, k=4, H=256, F=128)
    _run_layer_case(shape, 16, "zipf_rank", [1, 2, 4, 40], split=(0.0625, None, 1.0))


def test_layer_split_precision_device_orchestration():
    shape = W.reduced(SPLIT, E=32, k=8, H=256, F=128, layers=2)
    _run_layer_case(shape, 24, "zipf_rank", [1, 2, 1, 3], layers_order=[0, 1], device_plan=True,
                    split=(0.03125, [1.0, 2.0], 1.0))


def test_layer_split_precision_with_policy():
    shape = W.reduced(SPLIT, E=16, k=4, H=256, F=128, layers=2)
    _run_layer_case(shape, 12, "zipf_rank", [1, 3, 1, 2], layers_order=[0, 1],
                    policy=(B.MOE_POLICY_MRS, 4, None), split=(0.125, None, 0.5))


def test_layer_staging_prefill_stack():
    """Prefill steps at or above the threshold run from the two full-layer buffers (the next
    layer loads while the current one computes); decode steps in between use the decode cache,
    whose tables the staged steps leave alone."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    lay = _run_layer_case(shape, 14, "zipf_rank", [1, 24, 3, 40, 1], layers_order=[0, 1, 2],
                          staging=8)
    # first staged round: buffer 0 loads layer 0, then layers 1, 2, 0 are each prefetched
    # while the previous one computes; second round: 3 prefetches, every step a buffer hit
    assert lay.ctx.stage_counters() == {"staged_steps": 6, "stage_copies": 16 * 7}


def test_layer_staging_split_shared_rule_threshold():
    """The pages' switch, floor(resident slots / k), with split-precision experts and a
    shared expert: a single layer is loaded once and stays staged."""
    shape = W.reduced(SPLIT, E=16, k=4, H=256, F=128)
    lay = _run_layer_case(shape, 8, "zipf_rank", [1, 2, 4, 24, 1], staging=-1,
                          split=(0.125, None, 1.0))
    # 8 resident slots, k = 4: steps of T >= 2 are staged
    assert lay.ctx.stage_counters() == {"staged_steps": 3, "stage_copies": 16}


def test_split_and_staging_reject_bad_settings():
    """Split routing needs split-precision weights and finite constants; staging needs room
    for its buffers in the pool and excludes device orchestration."""
    shape = W.reduced(MIX, E=8, k=2, H=256, F=256)
    plain = Hn.SlotCacheLayer(shape, 4, W.initial_residency(shape, 4, "random"), 8)
    with pytest.raises(B.MoeError):
        plain.ctx.set_split(True, 0.1)  # bf16 weights
    plain.ctx.set_split(False)  # switching off is always allowed
    with pytest.raises(B.MoeError):
        plain.ctx.set_staging(True)  # the pool has no room for the staging buffers
    staged = Hn.SlotCacheLayer(shape, 4, W.initial_residency(shape, 4, "random"), 8, staging=True)
    staged.ctx.set_staging(True)
    with pytest.raises(B.MoeError):
        staged.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    staged.ctx.set_staging(False)
    staged.ctx.set_orchestration(B.MOE_ORCH_DEVICE)
    with pytest.raises(B.MoeError):
        staged.ctx.set_staging(True)
    with pytest.raises(B.MoeError):
        staged.ctx.set_staging(True, threshold=-2)
    sp = W.reduced(SPLIT, E=8, k=2, H=256, F=128)
    split = Hn.SlotCacheLayer(sp, 8, W.initial_residency(sp, 8, "identity"), 4)
    with pytest.raises(B.MoeError):
        split.ctx.set_split(True, float("nan"))
    with pytest.raises(B.MoeError):
        split.ctx.set_split(True, 0.1, beta=[float("inf")])
    split.ctx.set_split(True, 0.1, beta=[0.5], gamma=0.75)


def test_layer_shared_experts():
    shape = W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), E=16, k=6, H=256, F=256)
    _run_layer_case(shape, 8, "zipf_rank", [1, 32, 5])


def test_layer_int4_shared_expert_misses():
    shape = W.reduced(DSV3, E=32, k=8, H=256, F=128)
    _run_layer_case(shape, 12, "zipf_rank", [1, 6, 40, 2])


def test_layer_all_resident_decode_bf16_shared():
    """Every expert resident, with shared experts: decode steps of 1 to 8 tokens, whose
    routing front end (one launch up to 4 tokens, logits then one selecting workgroup
    beyond) writes the FFN's work list itself, so the FFN call runs without its plan."""
    shape = W.reduced(W.shape_of("dsv2lite_e64k6s2_h2048_f1408_bf16"), E=16, k=6, H=256, F=256)
    _run_layer_case(shape, 16, "zipf_rank", [1, 2, 4, 3, 8, 1])


def test_layer_all_resident_decode_int4_shared():
    shape = W.reduced(DSV3, E=16, k=4, H=256, F=128)
    _run_layer_case(shape, 16, "zipf_rank", [1, 4, 2, 7, 1])


def test_layer_mixtral_full_size_decode():
    """Full Mixtral-shaped layer (H=4096, F=14336), 4 of 8 experts resident, decode T=1 and T=8."""
    _run_layer_case(MIX, 4, "random", [1, 8])


def test_forward_steps_matches_single_calls():
    """moe_ctx_forward_steps runs the same steps as moe_layer_forward calls: same output, tables, counters."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    say(f"forward_steps {shape.name}")
    residency = W.initial_residency(shape, 14, "zipf_rank")
    a = Hn.SlotCacheLayer(shape, 14, residency, 4)
    b = Hn.SlotCacheLayer(shape, 14, residency, 4, store=a.store)
    oa = torch.empty(4, shape.H, dtype=torch.bfloat16, device=_dev())
    ob = torch.empty_like(oa)
    for step in range(5):
        T = 1 + step % 4
        xs = [(l, W.tokens(shape, T, layer=l, step=step, device=_dev())) for l in range(3)]
        for l, x in xs:
            a.forward(x, layer=l, out=oa[:T])
        b.forward_steps(xs, ob[:T])
        torch.cuda.synchronize()
        assert torch.equal(oa[:T], ob[:T])
    assert a.counters() == b.counters()
    ta, tb = a.tables(), b.tables()
    for u, v in zip(ta, tb):
        assert np.array_equal(np.asarray(u), np.asarray(v))
    assert a.err.item() == 0 and b.err.item() == 0


def test_prefetch_commit_overtaken_by_a_demand_fill_is_refused():
    """A prefetch copies expert A into slot 1 (tag 5) and is committed late; meanwhile a demand
    fill puts expert B into the same slot (tag 6, committed). The late commit of A finds tag 6
    and is refused: the table keeps B, A stays absent and the slot holds B's bytes. The order
    is forced from the host (each call completes before the next is issued)."""
    shape = W.reduced(MIX, E=6, k=2, H=256, F=128)
    store = Hn.ExpertStore(shape)
    S, E = 3, 6
    pool = torch.zeros(S * store.stride, dtype=torch.uint8, device=_dev())
    lut = torch.full((E,), -1, dtype=torch.int32, device=_dev())
    owner = torch.full((S,), -1, dtype=torch.int32, device=_dev())
    tags = torch.zeros(S, dtype=torch.int64, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    fs = torch.cuda.Stream()
    cs = torch.cuda.current_stream()
    A, B_ = 4, 2
    B.slot_prefetch(pool, store.stride, 1, store.host[A], store.stride, tags, 5, fs)
    torch.cuda.synchronize()
    assert tags.cpu().tolist() == [0, 5, 0] and lut.cpu().tolist() == [-1] * E  # copied, not committed
    B.slot_fill(pool, store.stride, 1, store.host[B_], store.stride, lut, B_, owner, tags, 6, err, fs, cs)
    torch.cuda.synchronize()
    B.slot_commit(lut, A, owner, 1, tags, 5, err)  # the prefetch's commit, now stale
    torch.cuda.synchronize()
    assert err.item() == B.MOE_ERR_STALE_TAG
    assert lut.cpu().tolist() == [-1, -1, 1, -1, -1, -1] and owner.cpu().tolist() == [-1, B_, -1]
    assert torch.equal(pool[store.stride:2 * store.stride].cpu(), store.host[B_])
    # an uncontested prefetch commits normally
    err.zero_()
    B.slot_prefetch(pool, store.stride, 0, store.host[A], store.stride, tags, 7, fs)
    fs.synchronize()
    B.slot_commit(lut, A, owner, 0, tags, 7, err)
    torch.cuda.synchronize()
    assert err.item() == 0 and lut.cpu().tolist()[A] == 0
    assert torch.equal(pool[:store.stride].cpu(), store.host[A])


@pytest.mark.parametrize("window_us,slots", [(1e6, 10), (5.0, 12), (0.0, 10)])  # all free, 1, none
def test_forward_steps_prefetch_next_layer(window_us, slots):
    """Miss prefetch inside a stack step (MoE-CORE summary page, Mechanism): each layer's step
    also evaluates the next layer's router on its own tokens and copies the top predicted
    non-resident experts ahead, as many as the window hides at the given bandwidth. The
    oracle's planner does the same (moe_layer, then prefetch with the oracle's own
    prediction) and its pool takes the same copies: outputs, tables and the prefetch
    count must agree after every stack step."""
    shape = W.reduced(W.shape_of("qwen3moe_l48_e128k8_h2048_f768_bf16"), layers=3, E=16, k=4, H=256,
                      F=128, blobs=16)
    L, E, k = shape.layers, shape.E, shape.k
    residency = W.initial_residency(shape, slots, "zipf_rank")
    lay = Hn.SlotCacheLayer(shape, slots, residency, t_max=3)
    bw = 50.0
    lay.ctx.set_prefetch(True, t_remain_us=0.0, t_attn_us=window_us, t_launch_us=0.0, bw_gbs=bw)
    wts = OracleWeights(shape)
    pool = O.SlotPool(slots, L, E)
    for s_, o_ in enumerate(residency):
        if o_ is not None:
            pool.commit(s_, o_[0], o_[1], wts.of(*o_))
    planner = O.LruSlotPlanner(slots, L, E, residency)
    n_pf = 0
    for step, T in enumerate([1, 2, 1, 3, 1, 2]):
        say(f"prefetch window={window_us} step={step} T={T}")
        xs = [W.tokens(shape, T, layer=l, step=step, device=_dev()) for l in range(L)]
        outs = [torch.empty(T, shape.H, dtype=torch.bfloat16, device=_dev()) for _ in range(L)]
        lay.ctx.forward_steps([(l, xs[l], *lay.routers[l], outs[l]) for l in range(L)], B.MOE_BF16)
        torch.cuda.synchronize()
        assert lay.err.item() == 0
        for l in range(L):
            wr, b = lay.routers[l]
            ref = O.moe_layer(xs[l], wr, b, k, layer=l, pool=pool, planner=planner,
                              weights_of_expert=lambda e, l=l: wts.of(l, e))
            r = rel_l2(outs[l].float().cpu().numpy(), ref["out"])
            assert r <= TOL[shape.wfmt], (step, l, r)
            if l + 1 < L:
                pr = O.route(xs[l], *lay.routers[l + 1], k)
                sc = O.step_scores(pr["logits"]).astype(np.float32)
                got = planner.prefetch(l + 1, pr["ids"], sc, window_us, bw, lay.stride)
                for e, s_ in got:
                    pool.commit(s_, l + 1, e, wts.of(l + 1, e))
                n_pf += len(got)
        lut_h, owner_h, last_use_h, clock_h = lay.tables()
        assert lay.lut.cpu().numpy().reshape(L, E).tolist() == planner.lut.tolist(), step
        assert lut_h.reshape(L, E).tolist() == planner.lut.tolist()
        assert last_use_h.tolist() == planner.last_use and clock_h == planner.clock
    pc = lay.ctx.prefetch_counters()
    say(f"  prefetched {pc}, oracle {n_pf}")
    assert pc["prefetched"] == n_pf
    if window_us >= 1e6:
        assert n_pf > 0
    if window_us == 0.0:
        assert n_pf == 0
