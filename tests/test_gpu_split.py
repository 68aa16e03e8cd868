"""GPU parity of split-precision experts (RapidMoE Algorithm 1 and Algorithm 3)
against the oracle: the step scores, the critical split and the expert FFN
over MOE_INT4G128_RESPLIT slots.

Bars: the critical mask is bit-exact (decided in float32 on both sides from
the kernel's own scores); step scores within 2e-6 relative of the oracle's
softmax; expert rows within 2e-2 relative L2 (the int4 bar), low-precision
rows bitwise equal to a MOE_INT4G128 call over the same slots.
"""
import numpy as np
import pytest
import torch

import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import harness as Hn
from expert_offload_routed_amd import workloads as W
from gpu_common import TOL, oracle_y_rows, rel_l2, say

pytestmark = pytest.mark.gpu

DSV3 = W.shape_of("dsv3_e256k8s1_h7168_f2048_int4")


def _dev():
    return torch.device("cuda:0")


def _split_shape(**kw):
    return W.reduced(DSV3, wfmt="int4g128_resplit", n_shared=0, **kw)


# ---------------------------------------------------------- scores, split --
@pytest.mark.parametrize("T,E", [(1, 8), (5, 64), (37, 256), (300, 1000)])
def test_step_scores_and_critical_split(T, E):
    say(f"split scores T={T} E={E}")
    g = torch.Generator().manual_seed(T * 1000 + E)
    logits = (torch.randn(T, E, generator=g) * 2.0).to(_dev())
    sc = B.moe_step_scores(logits, T, E)
    torch.cuda.synchronize()
    sc_h = sc.cpu().numpy()
    np.testing.assert_allclose(sc_h, O.step_scores(logits.cpu().numpy()), rtol=2e-6, atol=1e-8)
    distinct = np.sort(np.random.default_rng(E).choice(E, size=max(1, E // 3), replace=False))
    srt = np.sort(sc_h[distinct])
    # thresholds: none critical, all critical, a median split, and one equal to a score (>= holds)
    for th in (float(srt[-1]) * 2 + 1.0, 0.0, float(np.median(srt)), float(srt[len(srt) // 3])):
        m = B.moe_critical_split(sc, E, th)
        torch.cuda.synchronize()
        m = m.cpu().numpy().reshape(E)
        crit = set(O.critical_experts(sc_h, distinct, th))
        assert {int(e) for e in distinct if m[e] == 2} == crit
        assert all(m[e] in (1, 2) for e in range(E))
    # with an input mask: rows of groups to run, precision from the same scores
    rows = 3
    mask_in = torch.from_numpy(np.random.default_rng(T).integers(0, 2, (rows, E)).astype(np.int32)).to(_dev())
    th = float(np.median(srt))
    out = B.moe_critical_split(sc, E, th, mask_in=mask_in, rows=rows)
    torch.cuda.synchronize()
    mi, mo = mask_in.cpu().numpy(), out.cpu().numpy()
    want = np.where(mi == 0, 0, np.where(sc_h[None, :] >= np.float32(th), 2, 1))
    assert np.array_equal(mo, want)
    # in place
    B.moe_critical_split(sc, E, th, mask_in=mask_in, rows=rows, mask_out=mask_in)
    torch.cuda.synchronize()
    assert np.array_equal(mask_in.cpu().numpy(), want)


def test_critical_split_rejects_bad_args():
    sc = torch.zeros(4, device=_dev())
    with pytest.raises(B.MoeError):
        B.moe_critical_split(sc, 0, 0.1)
    with pytest.raises(B.MoeError):
        B.moe_step_scores(torch.zeros(4, 2000, device=_dev()), 4, 2000)


# --------------------------------------------------------------- expert FFN --
def _split_pool(shape, lut_perm):
    store = Hn.ExpertStore(shape)
    pool = torch.empty(shape.E * store.stride, dtype=torch.uint8, device=_dev())
    for e in range(shape.E):
        s = lut_perm[e]
        pool[s * store.stride:(s + 1) * store.stride].copy_(store.host[W.blob_of(shape, 0, e)])
    return pool, store.stride, torch.tensor(lut_perm, dtype=torch.int32, device=_dev())


SPLIT_FFN_CASES = [
    (_split_shape(E=16, k=4, H=512, F=256), 1),
    (_split_shape(E=16, k=4, H=512, F=256), 3),
    (_split_shape(E=16, k=4, H=512, F=256), 40),    # low groups on GEMV and MFMA tiles
    (_split_shape(E=16, k=4, H=512, F=256), 300),   # low groups on MFMA tiles; high groups of ~75 rows
    (_split_shape(E=8, k=4, H=384, F=384), 40),     # 3 scale groups per row, partial tiles
    (_split_shape(E=12, k=8, H=7168, F=2048), 2),   # full hidden/FFN sizes
    (_split_shape(E=12, k=8, H=7168, F=2048), 24),
    (_split_shape(E=12, k=8, H=7168, F=2048), 200),  # both precisions on MFMA tiles, 2 per group
]


@pytest.mark.parametrize("shape,T", SPLIT_FFN_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_expert_ffn_split_precision(shape, T):
    say(f"split ffn {shape.name} T={T}")
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    rng = np.random.default_rng(T + E)
    lut_perm = rng.permutation(E).tolist()
    pool, stride, lut = _split_pool(shape, lut_perm)
    x = W.tokens(shape, T, device=_dev())
    wr, b = W.router(shape, device=_dev())
    _, ids, _ = B.moe_route(x, wr, b, k)
    p = B.moe_permute(ids, E)
    ids_np = ids.cpu().numpy()
    ref = O.permute(ids_np, E)
    distinct = [int(e) for e in ref["distinct"]]
    # precision per expert: 0 skip (one routed expert), 1 low, 2 high, both present
    mask_np = rng.integers(1, 3, E).astype(np.int32)
    if len(distinct) >= 3:
        mask_np[distinct[0]], mask_np[distinct[1]], mask_np[distinct[2]] = 0, 1, 2
    mask = torch.from_numpy(mask_np).to(_dev())
    code = B.MOE_INT4G128_RESPLIT
    ws = torch.empty(B.moe_ffn_workspace_bytes(T, H, F, E, k, code), dtype=torch.uint8, device=_dev())
    err = torch.zeros(1, dtype=torch.int32, device=_dev())
    y = torch.full((T * k, H), 7.0, dtype=torch.float32, device=_dev())
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, mask, pool, stride, code, T, H, F, E, k, y, err, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    o = ref["offsets"]
    run = [e for e in distinct if mask_np[e] != 0]
    crit = {e for e in run if mask_np[e] == 2}
    yr = oracle_y_rows(shape, x, ids_np, ref["perm"], o, 0, run, critical=crit)
    y_h = y.cpu().numpy()
    rows = np.concatenate([np.arange(o[e], o[e + 1]) for e in run])
    r = rel_l2(y_h[rows], yr[rows])
    for e in (distinct[:3] if len(distinct) >= 3 else []):
        if mask_np[e] == 0:
            assert np.all(y_h[o[e]:o[e + 1]] == 7.0)
    hi_rows = [np.arange(o[e], o[e + 1]) for e in run if e in crit]
    lo_rows = [np.arange(o[e], o[e + 1]) for e in run if e not in crit]
    say(f"  rel L2 {r:.3e}; {len(crit)} high, {len(run) - len(crit)} low groups")
    assert r <= TOL[shape.wfmt]
    if hi_rows:
        hr = np.concatenate(hi_rows)
        say(f"  high rows rel L2 {rel_l2(y_h[hr], yr[hr]):.3e}")
        assert rel_l2(y_h[hr], yr[hr]) <= TOL[shape.wfmt]
    # low rows: what the int4 path computes on the same slots. With one token both take
    # the same GEMV, so bit for bit; with more, the int4 path runs groups of up to 32 rows
    # on the MFMA GEMV while split-precision steps keep the GEMV and the MFMA tiles, which
    # fold the same exact group sums in another fp32 order (a few int8 codes of h flip)
    if lo_rows:
        lr = np.concatenate(lo_rows)
        lo_mask = torch.from_numpy(np.where(mask_np == 1, 1, 0).astype(np.int32)).to(_dev())
        y4 = torch.full_like(y, 7.0)
        ws4 = torch.empty(B.moe_ffn_workspace_bytes(T, H, F, E, k, B.MOE_INT4G128), dtype=torch.uint8,
                          device=_dev())
        B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, lo_mask, pool, stride, B.MOE_INT4G128, T, H, F,
                         E, k, y4, err, ws4)
        torch.cuda.synchronize()
        if T == 1:
            assert torch.equal(y[lr], y4[lr])
        else:
            d = rel_l2(y_h[lr], y4.cpu().numpy()[lr])
            say(f"  low rows vs the int4 path: rel L2 {d:.3e}")
            assert d <= 5e-3
    # no mask: every group at high precision; determinism of the high rows
    y2 = torch.full_like(y, 7.0)
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, code, T, H, F, E, k, y2, err, ws)
    torch.cuda.synchronize()
    if hi_rows:
        assert torch.equal(y2[hr], y[hr])
    ya = oracle_y_rows(shape, x, ids_np, ref["perm"], o, 0, distinct, critical=None)
    ra = rel_l2(y2.cpu().numpy(), ya)
    say(f"  all-high rel L2 {ra:.3e}")
    assert ra <= TOL[shape.wfmt]
