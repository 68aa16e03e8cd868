"""Pins of the oracle to things other than itself (CPU only).

Every check goes through a different route than the oracle's own code: brute
force on tiny inputs, closed forms worked out by hand, an independent library
routine (scipy, torch.nn.functional, numpy's stable argsort), a textbook
algorithm the policy reduces to, or an invariant the definition implies.
"""
import math
from collections import OrderedDict

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as Fnn

import hand_cases as HC
import oracle as O
from expert_offload_routed_amd import workloads as W


# ------------------------------------------------------------ router logits --
def test_router_logits_closed_form():
    # x = [1, 2]; rows of w_r are expert vectors; bias shifts each logit.
    x = np.array([[1.0, 2.0], [0.0, -1.0]])
    w_r = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    b = np.array([0.5, -0.5, 0.0])
    got = O.router_logits(x, w_r, b)
    assert got.tolist() == [[1.5, 1.5, 3.0], [0.5, -1.5, -1.0]]


def test_router_logits_matches_torch_linear_nonsquare():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(5, 37, generator=g, dtype=torch.float64)
    w = torch.randn(11, 37, generator=g, dtype=torch.float64)
    b = torch.randn(11, generator=g, dtype=torch.float64)
    ref = Fnn.linear(x, w, b).numpy()
    np.testing.assert_allclose(O.router_logits(x.numpy(), w.numpy(), b.numpy()), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- selection --
def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 6), (9, 9), (33, 8)])
def test_select_topk_equals_full_sort_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    scores = rng.integers(-3, 4, size=(40, E)).astype(np.float32)  # many exact ties
    ids = O.select_topk(scores, k)
    for t in range(scores.shape[0]):
        assert ids[t].tolist() == _brute_topk(scores[t], k)


def test_select_topk_hand_ties():
    s = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0], [-1.0, -0.0, 0.0, 5.0]], np.float32)
    assert O.select_topk(s, 2).tolist() == [[1, 2], [0, 1], [3, 1]]


def test_topk_margin_brute():
    rng = np.random.default_rng(3)
    s = rng.normal(size=(10, 12))
    m = O.topk_margin(s, 3)
    for t in range(10):
        v = sorted(s[t], reverse=True)
        assert m[t] == v[2] - v[3]
    assert np.all(np.isinf(O.topk_margin(s, 12)))


# ------------------------------------------------------------------ gating --
def test_gate_weights_two_experts_closed_form():
    l = np.array([[2.0, -1.0, 0.5]])
    ids = np.array([[0, 2]])
    w = O.gate_weights(l, ids, renorm=True)
    w0 = 1.0 / (1.0 + math.exp(0.5 - 2.0))  # softmax of two logits = logistic of the gap
    assert w[0, 0] == pytest.approx(w0, rel=1e-15)
    assert w[0, 1] == pytest.approx(1.0 - w0, rel=1e-14)


def test_gate_weights_against_scipy_softmax():
    rng = np.random.default_rng(4)
    l = rng.normal(size=(20, 16)) * 3
    ids = O.select_topk(l.astype(np.float32), 5)
    w = O.gate_weights(l, ids, renorm=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    sel = np.take_along_axis(l, ids, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13)
    w_raw = O.gate_weights(l, ids, renorm=False)
    np.testing.assert_allclose(w_raw, np.take_along_axis(scipy.special.softmax(l, axis=1), ids, axis=1),
                               rtol=1e-13)


def test_gate_weights_k_equals_e_is_plain_softmax_and_k1_is_one():
    rng = np.random.default_rng(5)
    l = rng.normal(size=(7, 6))
    ids = O.select_topk(l.astype(np.float32), 6)
    w = O.gate_weights(l, ids)
    np.testing.assert_allclose(w, np.take_along_axis(scipy.special.softmax(l, axis=1), ids, axis=1),
                               rtol=1e-13)
    w1 = O.gate_weights(l, O.select_topk(l.astype(np.float32), 1))
    assert np.all(w1 == 1.0)


def test_route_orders_by_descending_weight():
    s = W.shape_of("tiny_e8k2_h256_f512_fp32")
    r = O.route(W.tokens(s, 16), *W.router(s), k=2)
    assert np.all(np.diff(r["weights"], axis=1) <= 0)


# ------------------------------------------------------------- permutation --
@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 8, 2), (16, 8, 2), (37, 64, 6), (200, 256, 8)])
def test_permute_against_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32).reshape(T, k)
    p = O.permute(ids, E)
    flat = ids.reshape(-1)
    assert p["perm"].tolist() == np.argsort(flat, kind="stable").tolist()
    bc = np.bincount(flat, minlength=E)
    assert p["counts"].tolist() == bc.tolist()
    assert p["offsets"].tolist() == [0] + np.cumsum(bc).tolist()
    assert int(p["counts"].sum()) == T * k
    if T:
        assert np.array_equal(p["inv"][p["perm"]], np.arange(T * k))
    assert p["distinct"].tolist() == [e for e in range(E) if bc[e] > 0]
    # inside an expert's segment, tokens rise strictly (each token picks an expert once)
    for e in range(E):
        seg = p["perm"][p["offsets"][e]:p["offsets"][e + 1]] // k
        assert np.all(np.diff(seg) > 0)


# ------------------------------------------------------------- expert FFN ---
def test_swiglu_closed_form():
    x = np.array([[1.0, 2.0]])
    gate = np.array([[1.0, 0.0]])   # g = x0 = 1
    up = np.array([[0.0, 1.0]])     # u = x1 = 2
    down = np.array([[1.0], [-1.0]])
    s1 = 1.0 / (1.0 + math.exp(-1.0))  # SiLU(1) = 1 * sigmoid(1)
    y = O.swiglu_expert(x, gate, up, down)
    assert y[0, 0] == pytest.approx(2 * s1, rel=1e-15)
    assert y[0, 1] == pytest.approx(-2 * s1, rel=1e-15)


def test_swiglu_matches_torch_nonsquare():
    g = torch.Generator().manual_seed(7)
    H, F, n = 24, 40, 5
    x = torch.randn(n, H, generator=g, dtype=torch.float64)
    gate = torch.randn(F, H, generator=g, dtype=torch.float64)
    up = torch.randn(F, H, generator=g, dtype=torch.float64)
    down = torch.randn(H, F, generator=g, dtype=torch.float64)
    ref = Fnn.linear(Fnn.silu(Fnn.linear(x, gate)) * Fnn.linear(x, up), down).numpy()
    got = O.swiglu_expert(x.numpy(), gate.numpy(), up.numpy(), down.numpy())
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- int4 and int8 ---
def _pack_int4(q):
    """Reference packer: two's-complement nibbles, even column in the low nibble."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def test_int4_decode_roundtrip_all_codes():
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, size=(6, 256))
    q[0, :16] = np.arange(-8, 8)
    assert np.array_equal(O.decode_int4(_pack_int4(q)), q.astype(np.int8))


def test_int4_dequant_group_boundaries():
    rows, K = 3, 384
    q = np.ones((rows, K), dtype=np.int64)
    q[:, 1::2] = -2
    scales = torch.tensor([[0.5, 0.25, 2.0], [1.0, 3.0, -0.125], [4.0, 0.0, 1.5]], dtype=torch.bfloat16)
    w = O.dequant_int4g128(_pack_int4(q), scales)
    s = scales.float().numpy().astype(np.float64)
    for r in range(rows):
        for c in (0, 1, 126, 127, 128, 129, 255, 256, 383):
            assert w[r, c] == q[r, c] * s[r, c // 128]


def test_int8_rows_error_bound_and_extremes():
    rng = np.random.default_rng(9)
    a = (rng.normal(size=(8, 300)) * rng.uniform(0.01, 50, size=(8, 1))).astype(np.float32)
    a[3] = 0.0
    q, s = O.quantize_rows_int8(a)
    assert q[3].tolist() == [0] * 300 and s[3] == 1.0
    for r in range(8):
        if r == 3:
            continue
        amax = np.abs(a[r]).max()
        assert s[r] == np.float32(amax / np.float32(127))
        assert np.abs(q[r]).max() == 127
        err = np.abs(a[r].astype(np.float64) - q[r].astype(np.float64) * float(s[r]))
        assert err.max() <= float(s[r]) * 0.5 * (1 + 1e-6)
    qn, sn = O.quantize_rows_int8(-a)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_w4a8_expert_close_to_dense_on_dequantised_weights():
    sh = W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), H=256, F=128)
    w = W.expert_weights(sh, 0)
    x = W.tokens(sh, 4).float().numpy()
    dense = O.swiglu_expert(x, O.dequant_int4g128(w["gate_q"], w["gate_s"]),
                            O.dequant_int4g128(w["up_q"], w["up_s"]),
                            O.dequant_int4g128(w["down_q"], w["down_s"]))
    q = O.swiglu_expert_w4a8(x, w)
    rel = np.linalg.norm(q - dense) / np.linalg.norm(dense)
    assert 0 < rel < 0.03  # only the two int8 activation roundings differ


def test_int8_rows_half_steps_round_to_even():
    # absmax 254 gives s = 2 exactly; 5/2, 3/2, -5/2, 1/2, -3/2 sit on half steps
    a = np.array([[254.0, 5.0, 3.0, -5.0, 1.0, -3.0, 7.0, 0.0]], np.float32)
    q, s = O.quantize_rows_int8(a)
    assert s.tolist() == [2.0]
    assert q.tolist() == [[127, 2, 2, -2, 0, -2, 4, 0]]


@pytest.mark.parametrize("H,F", [(128, 128), (512, 256)])
def test_w4a8_expert_exposes_requantised_h_by_hand(H, F):
    # tests/hand_cases.py: gate and up read single inputs, down is the identity, so
    # y = h_hat, the int8 requantisation of h, and the values are worked out by hand there
    # (half steps of x and of h round to even; one scale per row).
    w = HC.w4a8_expert(H, F)
    y = O.swiglu_expert_w4a8(HC.tokens(4, H), w)
    assert y[0, :14].tolist() == [127, 2, 4, -2, 126, 0, 2, -2, -8, 2, 2, 4, -2, 2]
    assert y.tolist() == HC.expected_y(4, H, F).tolist()
    assert y[1].tolist() == (4 * y[0]).tolist()


# ---------------------------------------------------------------- combine ---
def test_combine_linearity_and_zero_weight_poison():
    rng = np.random.default_rng(10)
    y = rng.normal(size=(4, 3, 8))
    w = np.zeros((4, 3))
    w[:, 1] = 1.0
    np.testing.assert_array_equal(O.combine(y, w), y[:, 1])
    y[:, 2] = np.nan
    w2 = np.array([[0.6, 0.4, 0.0]] * 4)
    out = O.combine(y, w2)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, 0.6 * y[:, 0] + 0.4 * y[:, 1], rtol=1e-15)
    sh = rng.normal(size=(2, 4, 8))
    np.testing.assert_allclose(O.combine(y, w2, sh), out + sh[0] + sh[1], rtol=1e-15)


# ---------------------------------------------------------- full layer ------
def _tiny_layer(lut_perm, E=8, k=2, H=64, F=96, T=12, **kw):
    sh = W.reduced(W.shape_of("tiny_e8k2_h256_f512_fp32"), E=E, k=k, H=H, F=F)
    x = W.tokens(sh, T)
    wr, b = W.router(sh)
    experts = [W.expert_weights(sh, e) for e in range(E)]
    pool = O.SlotPool(E, 1, E)
    for e in range(E):
        pool.commit(lut_perm[e], 0, e, experts[e])
    return O.moe_layer(x, wr, b, k, layer=0, pool=pool, planner=None,
                       weights_of_expert=lambda e: experts[e], **kw), experts, x, wr, b


def test_slot_relabel_invariance():
    a, *_ = _tiny_layer(list(range(8)))
    b, *_ = _tiny_layer([5, 2, 7, 0, 3, 6, 1, 4])
    assert np.array_equal(a["out"], b["out"])


def test_layer_e1_k1_is_dense_swiglu():
    res, experts, x, wr, b = _tiny_layer([0], E=1, k=1)
    w = {n: torch.tensor(t.numpy(), dtype=torch.float64) for n, t in experts[0].items()}
    xt = torch.tensor(x.numpy(), dtype=torch.float64)
    ref = Fnn.linear(Fnn.silu(Fnn.linear(xt, w["gate"])) * Fnn.linear(xt, w["up"]), w["down"]).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_layer_weighted_sum_by_hand():
    res, experts, x, wr, b = _tiny_layer(list(range(8)), T=3)
    ids, w = res["route"]["ids"], res["route"]["weights"]
    for t in range(3):
        acc = 0
        for j in range(2):
            e = experts[ids[t, j]]
            acc = acc + w[t, j] * O.swiglu_expert(x[t:t + 1].numpy(), e["gate"], e["up"], e["down"])[0]
        np.testing.assert_allclose(res["out"][t], acc, rtol=1e-13, atol=1e-15)


def _hand_expert(seed, H, F):
    g = np.random.default_rng(seed)
    return {"gate": g.normal(size=(F, H)) * 0.3, "up": g.normal(size=(F, H)) * 0.3,
            "down": g.normal(size=(H, F)) * 0.3}


def _dense_token(x_t, w):
    xt = torch.tensor(np.asarray(x_t, np.float64))
    t = {n: torch.tensor(v) for n, v in w.items()}
    return Fnn.linear(Fnn.silu(Fnn.linear(xt, t["gate"])) * Fnn.linear(xt, t["up"]), t["down"]).numpy()


def test_layer_two_waves_by_hand():
    # 2 slots, 4 experts. Slot 0 holds expert 0, slot 1 expert 3. Router = identity, so
    # token 0 = [3, 2, 0, 0] routes to (0, 1) and token 1 = [1, 0, 4, 0] to (2, 0).
    # U = {0, 1, 2}: hit 0 (slot 0), misses 1, 2; one victim (slot 1) -> wave 1 computes
    # 0 and 1 (1 filled into slot 1), wave 2 computes 2, filled into slot 0, which held
    # expert 0 in wave 1.
    H, F, E, k = 4, 3, 4, 2
    experts = [_hand_expert(40 + e, H, F) for e in range(E)]
    x = np.array([[3.0, 2.0, 0.0, 0.0], [1.0, 0.0, 4.0, 0.0]], np.float32)
    wr = np.eye(E, H, dtype=np.float32)
    pool = O.SlotPool(2, 1, E)
    pool.commit(0, 0, 0, experts[0])
    pool.commit(1, 0, 3, experts[3])
    planner = O.LruSlotPlanner(2, 1, E, residency=[(0, 0), (0, 3)])
    res = O.moe_layer(x, wr, None, k, layer=0, pool=pool, planner=planner,
                      weights_of_expert=lambda e: experts[e])
    assert res["route"]["ids"].tolist() == [[0, 1], [2, 0]]
    assert [(wv.compute, wv.fills) for wv in res["waves"]] == [([0, 1], [(1, 1)]), ([2], [(2, 0)])]
    assert pool.lut[0].tolist() == [-1, 1, 0, -1]
    assert pool.owner == [(0, 2), (0, 1)]
    wts = res["route"]["weights"]
    for t in range(2):
        want = sum(wts[t, j] * _dense_token(x[t], experts[res["route"]["ids"][t, j]]) for j in range(k))
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("S,T,resident", [(3, 40, 2), (1, 9, 0), (4, 25, 4)])
def test_layer_more_routed_than_slots_equals_direct_indexing(S, T, resident):
    sh = W.reduced(W.shape_of("tiny_e8k2_h256_f512_fp32"), H=64, F=96, zipf_s=None)
    x = W.tokens(sh, T)
    wr, b = W.router(sh)
    experts = [W.expert_weights(sh, e) for e in range(sh.E)]
    pool = O.SlotPool(S, 1, sh.E)
    own = [(0, e) for e in (5, 1, 6, 2)[:resident]] + [None] * (S - resident)
    for s, o in enumerate(own):
        if o is not None:
            pool.commit(s, 0, o[1], experts[o[1]])
    planner = O.LruSlotPlanner(S, 1, sh.E, residency=own)
    res = O.moe_layer(x, wr, b, sh.k, layer=0, pool=pool, planner=planner,
                      weights_of_expert=lambda e: experts[e])
    U = res["perm"]["distinct"]
    assert len(U) > S and len(res["waves"]) >= 2
    ids, wts = res["route"]["ids"], res["route"]["weights"]
    xs = O.as_f64(x)
    for t in range(T):
        want = sum(wts[t, j] * _dense_token(xs[t], {n: O.as_f64(v) for n, v in experts[ids[t, j]].items()})
                   for j in range(sh.k))
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-11, atol=1e-13)
    # the table after the last wave is what the pool holds: every resident entry points
    # at a slot whose contents are that expert
    for e in range(sh.E):
        s = pool.lut[0, e]
        if s >= 0:
            assert pool.content[s] is experts[e]


def test_layer_sampled_rows_are_the_full_rows():
    full, *_ = _tiny_layer(list(range(8)), T=12)
    rows = [0, 5, 11]
    part, *_ = _tiny_layer(list(range(8)), T=12, rows=rows)
    assert np.array_equal(part["out"][rows], full["out"][rows])
    assert not np.any(part["out"][[t for t in range(12) if t not in rows]])
    assert np.array_equal(part["route"]["ids"], full["route"]["ids"])


def test_layer_critical_set_picks_the_precision_per_expert():
    sh = W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), E=4, k=2, H=256, F=128,
                   wfmt="int4g128_resplit", zipf_s=None)
    g = np.random.default_rng(21)
    masters = [[g.normal(size=s) * 0.02 for s in ((128, 256), (128, 256), (256, 128))] for _ in range(4)]
    experts = [O.resplit_expert(*m) for m in masters]
    x = W.tokens(sh, 6)
    wr, b = W.router(sh)
    pool = O.SlotPool(4, 1, 4)
    for e in range(4):
        pool.commit(e, 0, e, experts[e])
    crit = {1, 3}
    res = O.moe_layer(x, wr, b, 2, layer=0, pool=pool, planner=None,
                      weights_of_expert=lambda e: experts[e], critical=crit)
    ids, wts = res["route"]["ids"], res["route"]["weights"]
    for t in range(6):
        want = sum(wts[t, j] * O.swiglu_expert_split(O.as_f32(x)[t:t + 1], experts[ids[t, j]],
                                                     int(ids[t, j]) in crit)[0] for j in range(2))
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------- LRU slot planner ---
def test_planner_reduces_to_textbook_lru_for_single_expert_requests():
    rng = np.random.default_rng(11)
    E, S = 12, 4
    planner = O.LruSlotPlanner(S, 1, E)
    lru = OrderedDict()
    for step in range(400):
        e = int(rng.zipf(1.3) - 1) % E
        before = planner.lut[0, e] >= 0
        waves = planner.plan(0, [e])
        # textbook LRU cache of capacity S
        hit = e in lru
        if hit:
            lru.move_to_end(e)
        else:
            if len(lru) == S:
                lru.popitem(last=False)
            lru[e] = True
        assert before == hit, step
        assert sorted(int(v) for v in np.flatnonzero(planner.lut[0] >= 0)) == sorted(lru)
        assert len(waves) == 1 and len(waves[0].fills) == (0 if hit else 1)


def test_planner_hand_trace():
    # 3 slots, one layer of 6 experts; slot 2 starts empty.
    p = O.LruSlotPlanner(3, 1, 6, residency=[(0, 4), (0, 1), None])
    w = p.plan(0, [1, 3])          # hit 1 (slot 1); miss 3 -> empty slot 2
    assert [(x.compute, x.fills) for x in w] == [([1, 3], [(3, 2)])]
    w = p.plan(0, [0, 3])          # hit 3; miss 0 -> LRU among {0 (last 0), 1 (last 1)} = slot 0
    assert [(x.compute, x.fills) for x in w] == [([0, 3], [(0, 0)])]
    assert p.lut[0].tolist() == [0, 1, -1, 2, -1, -1]
    w = p.plan(0, [1, 2, 4, 5])    # |U| = 4 > S = 3: hit 1 stays; misses 2, 4, 5
    # wave 1: hit 1 + first two misses into victims by LRU: slot 0 (last 2) vs 2 (last 2) -> id order 0, 2
    assert [(x.compute, x.fills) for x in w] == [([1, 2, 4], [(2, 0), (4, 2)]), ([5], [(5, 0)])]
    assert p.lut[0].tolist() == [-1, 1, -1, -1, 2, 0]
    assert p.last_use == [3, 3, 3]


def test_planner_invariants_random_multilayer():
    rng = np.random.default_rng(12)
    L, E, S, k = 3, 10, 7, 3
    p = O.LruSlotPlanner(S, L, E)
    for step in range(300):
        layer = step % L
        T = int(rng.integers(1, 5))
        U = sorted({int(e) for e in rng.choice(E, size=(T * k), replace=True)})
        lut_before = p.lut.copy()
        hits = [e for e in U if lut_before[layer, e] >= 0]
        waves = p.plan(layer, U)
        computed = [e for wv in waves for e in wv.compute]
        assert sorted(computed) == U
        fills = [f for wv in waves for f in wv.fills]
        assert sorted(e for e, _ in fills) == sorted(set(U) - set(hits))
        # wave 1's fills never land on a slot holding a hit of this call
        kept = {int(lut_before[layer, e]) for e in hits}
        assert not kept & {s for _, s in waves[0].fills}
        # no slot is filled twice within one wave
        for wv in waves:
            assert len({s for _, s in wv.fills}) == len(wv.fills)
        # table is injective and the owner list is its inverse
        own = {}
        for (l_, e_), s in np.ndenumerate(p.lut):
            if s >= 0:
                assert s not in own
                own[int(s)] = (l_, e_)
        for s in range(S):
            assert p.owner[s] == own.get(s)
        if len(U) <= S:
            assert all(p.lut[layer, e] >= 0 for e in U)


# ----------------------------------------------------- eviction scores ---
def _trace(rng, L, E, k, steps):
    out = []
    for step in range(steps):
        layer = step % L
        T = int(rng.integers(1, 4))
        logits = rng.normal(size=(T, E))
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        out.append((layer, sorted({int(e) for e in ids.ravel()}), logits))
    return out


def test_step_scores_is_mean_softmax():
    lg = np.array([[0.0, 1.0, -2.0], [3.0, 3.0, 0.5]])
    want = scipy.special.softmax(lg, axis=1).mean(axis=0)
    np.testing.assert_allclose(O.step_scores(lg), want, rtol=1e-15)
    assert O.step_scores(lg).sum() == pytest.approx(1.0, abs=1e-15)


@pytest.mark.parametrize("policy", ["mrs_w1", "fresh_only"])
def test_scored_planner_reduces_to_lru(policy):
    # MRS over a window of one step is 0 for every expert, and the routing-history
    # score with only the freshness weight orders a single layer by last selection:
    # both leave the (last use, slot id) order of plain LRU.
    rng = np.random.default_rng(21)
    L, E, S, k = (3 if policy == "mrs_w1" else 1), 9, 5, 2
    pol = (O.MinusRecentScore(L, E, 1) if policy == "mrs_w1"
           else O.RoutingHistoryScore(L, E, 4, weights=(0.0, 0.0, 0.0, 1.0), lam=0.5))
    a = O.ScoredSlotPlanner(S, L, E, pol)
    b = O.LruSlotPlanner(S, L, E)
    for layer, U, logits in _trace(rng, L, E, k, 300):
        wa = a.plan(layer, U, O.step_scores(logits))
        wb = b.plan(layer, U)
        assert [(w.compute, w.fills) for w in wa] == [(w.compute, w.fills) for w in wb]
        assert np.array_equal(a.lut, b.lut)


def test_mrs_hand_trace():
    # 2 slots holding experts 0 and 1; window of 3 steps.
    p = O.ScoredSlotPlanner(2, 1, 3, O.MinusRecentScore(1, 3, 3), residency=[(0, 0), (0, 1)])
    assert p.plan(0, [0], [0.6, 0.1, 0.3])[0].fills == []
    assert p.plan(0, [1], [0.5, 0.4, 0.1])[0].fills == []
    # miss 2: MRS(0) = 0.6+0.5+0.2-0.2 = 1.1, MRS(1) = 0.1+0.4+0.1-0.1 = 0.5 -> slot 1 goes
    # (plain LRU would take slot 0: expert 0 was last used one step earlier than expert 1)
    assert p.plan(0, [2], [0.2, 0.1, 0.7])[0].fills == [(2, 1)]
    # miss 1: window is now steps 2..4: MRS(0) = 0.5+0.2+0.1-0.1 = 0.7, MRS(2) = 0.1+0.7+0.1-0.1 = 0.8
    assert p.plan(0, [1], [0.1, 0.8, 0.1])[0].fills == [(1, 0)]
    assert p.lut[0].tolist() == [-1, 0, 1]


def test_history_count_only_hand_trace():
    # count over a 4-step window: expert 0 was picked twice, expert 1 once but later
    def run(planner):
        fills = []
        for U in ([0], [0], [1], [2]):
            fills.append(planner.plan(0, U, [1 / 3] * 3)[0].fills if isinstance(planner, O.ScoredSlotPlanner)
                         else planner.plan(0, U)[0].fills)
        return fills
    scored = O.ScoredSlotPlanner(2, 1, 3, O.RoutingHistoryScore(1, 3, 4, weights=(1.0, 0.0, 0.0, 0.0)),
                                 residency=[(0, 0), (0, 1)])
    lru = O.LruSlotPlanner(2, 1, 3, residency=[(0, 0), (0, 1)])
    assert run(scored)[-1] == [(2, 1)]   # the less often picked expert 1 goes
    assert run(lru)[-1] == [(2, 0)]      # LRU drops the older expert 0


def test_history_ema_closed_form():
    lam, E = 0.8, 4
    pol = O.RoutingHistoryScore(1, E, 3, lam=lam)
    picks = [[0, 2], [1], [0], [], [0, 3], [2]]
    for U in picks:
        pol.observe(0, np.full(E, 0.25), U)
    n = len(picks)
    for e in range(E):
        want = sum((1 - lam) * lam ** (n - 1 - i) for i, U in enumerate(picks) if e in U)
        assert pol.ema[0][e] == pytest.approx(want, rel=1e-14, abs=1e-15)
    # age since last selection and the window count, by hand
    assert [n - pol.last[0][e] for e in range(E)] == [1, 4, 0, 1]
    cnt, _, _, age = pol._features(0)
    assert cnt == [1.0, 0.0, 1.0, 1.0] and age == [1.0, 4.0, 0.0, 1.0]


@pytest.mark.parametrize("policy", ["mrs", "history"])
def test_scored_plans_invariant_under_power_of_two_score_scale(policy):
    rng = np.random.default_rng(22)
    L, E, S, k = 2, 8, 5, 2
    mk = (lambda: O.MinusRecentScore(L, E, 5)) if policy == "mrs" else \
        (lambda: O.RoutingHistoryScore(L, E, 5, weights=(0.5, 1.0, 2.0, 0.25), lam=0.75))
    a, b = O.ScoredSlotPlanner(S, L, E, mk()), O.ScoredSlotPlanner(S, L, E, mk())
    for layer, U, logits in _trace(rng, L, E, k, 200):
        sc = O.step_scores(logits).astype(np.float32)
        wa, wb = a.plan(layer, U, sc), b.plan(layer, U, sc * np.float32(4.0))
        assert [(w.compute, w.fills) for w in wa] == [(w.compute, w.fills) for w in wb]


def test_scored_planner_invariants_random_multilayer():
    rng = np.random.default_rng(23)
    L, E, S, k = 3, 10, 7, 3
    p = O.ScoredSlotPlanner(S, L, E, O.RoutingHistoryScore(L, E, 6))
    for layer, U, logits in _trace(rng, L, E, k, 300):
        lut_before = p.lut.copy()
        hits = [e for e in U if lut_before[layer, e] >= 0]
        waves = p.plan(layer, U, O.step_scores(logits))
        assert sorted(e for wv in waves for e in wv.compute) == U
        fills = [f for wv in waves for f in wv.fills]
        assert sorted(e for e, _ in fills) == sorted(set(U) - set(hits))
        kept = {int(lut_before[layer, e]) for e in hits}
        assert not kept & {s for _, s in waves[0].fills}
        for s in range(S):
            o = p.owner[s]
            assert o is None or p.lut[o] == s
        if len(U) <= S:
            assert all(p.lut[layer, e] >= 0 for e in U)


# ------------------------------------------------ split-precision experts ---
def test_round_bf16_matches_torch_including_ties():
    rng = np.random.default_rng(31)
    a = rng.normal(size=4096).astype(np.float32) * np.float32(3.0)
    hi = rng.integers(0, 1 << 16, size=512, dtype=np.uint32) << 16
    ties = (hi | np.uint32(0x8000)).view(np.float32)            # exactly halfway
    ties = ties[np.isfinite(ties)]
    for v in (a, ties):
        want = torch.tensor(v).to(torch.bfloat16).to(torch.float32).numpy()
        np.testing.assert_array_equal(O.round_bf16(v), want)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantize_sym_g128_bounds(bits):
    rng = np.random.default_rng(32 + bits)
    w = (rng.normal(size=(6, 512)) * 0.02).astype(np.float32)
    w[2, 128:256] = 0.0                                     # an all-zero group
    q, s = O.quantize_sym_g128(w, bits)
    qmax = 2 ** (bits - 1) - 1
    g = w.reshape(6, 4, 128)
    absmax = np.abs(g).max(axis=2)
    want_s = torch.tensor(absmax / np.float32(qmax)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(s, want_s)
    assert q.min() >= -qmax - 1 and q.max() <= qmax
    assert not q.reshape(6, 4, 128)[2, 1].any() and s[2, 1] == 0
    recon = q.reshape(6, 4, 128).astype(np.float64) * s[:, :, None]
    err = np.abs(recon - g)
    clipped = np.abs(q.reshape(6, 4, 128)) >= qmax
    assert np.all(err[~clipped] <= s[:, :, None].repeat(128, 2)[~clipped] * 0.5 * (1 + 1e-6))
    # the largest element of every nonzero group lands on the edge of the code range
    edge = np.abs(q.reshape(6, 4, 128)).max(axis=2)
    assert set(np.unique(edge[absmax > 0]).tolist()) <= {qmax, qmax + 1}


def test_resplit_residual_and_dual_down():
    rng = np.random.default_rng(34)
    H, F = 256, 128
    gate = (rng.normal(size=(F, H)) * 0.02).astype(np.float32)
    up = (rng.normal(size=(F, H)) * 0.02).astype(np.float32)
    down = (rng.normal(size=(H, F)) * 0.02).astype(np.float32)
    w = O.resplit_expert(gate, up, down)
    for name, W in (("gate", gate), ("up", up)):
        wq = w[name + "_q"].astype(np.float64) * np.repeat(w[name + "_s"], 128, 1)
        wr = w[name + "_rq"].astype(np.float64) * np.repeat(w[name + "_rs"], 128, 1)
        e_low = np.abs(W - wq).mean()
        e_high = np.abs(W - (wq + wr)).mean()
        assert e_high < e_low / 8                         # the residual compensates the error
        assert np.all(np.abs(W - (wq + wr)) <= np.repeat(w[name + "_rs"], 128, 1) * 0.5 * (1 + 1e-6) + 1e-12)
    assert np.array_equal(w["down_lq"], O.quantize_sym_g128(down, 4)[0])
    dh = w["down_hq"].astype(np.float64) * np.repeat(w["down_hs"], 128, 1)
    dl = w["down_lq"].astype(np.float64) * np.repeat(w["down_ls"], 128, 1)
    assert np.abs(down - dh).mean() < np.abs(down - dl).mean() / 8


def test_critical_threshold_and_set():
    assert O.critical_threshold(0.1, 2.0, "prefill", 1.5) == pytest.approx(0.2)
    assert O.critical_threshold(0.1, 2.0, "decode", 1.5) == pytest.approx(0.3)
    scores = np.array([0.05, 0.30, 0.15, 0.29999], dtype=np.float32)
    assert O.critical_experts(scores, [0, 1, 2, 3], 0.0) == [0, 1, 2, 3]
    assert O.critical_experts(scores, [0, 1, 2, 3], 1.01) == []
    assert O.critical_experts(scores, [1, 2, 3], 0.3) == [1]        # >= includes the boundary
    assert O.critical_experts(scores, [0, 2], 0.1) == [2]           # only routed experts


def _pack_codes(q):
    """int8 codes [rows, K] -> packed signed nibbles [rows, K/2] (even index low)."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def test_split_low_path_is_the_int4_expert_and_high_path_closer_to_dense():
    rng = np.random.default_rng(35)
    H, F, T = 256, 128, 5
    gate, up, down = ((rng.normal(size=s) * 0.05).astype(np.float32) for s in ((F, H), (F, H), (H, F)))
    w = O.resplit_expert(gate, up, down)
    x = rng.normal(size=(T, H)).astype(np.float32)
    low = O.swiglu_expert_split(x, w, critical=False)
    w4 = {"gate_q": _pack_codes(w["gate_q"]), "gate_s": w["gate_s"], "up_q": _pack_codes(w["up_q"]),
          "up_s": w["up_s"], "down_q": _pack_codes(w["down_lq"]), "down_s": w["down_ls"]}
    np.testing.assert_array_equal(low, O.swiglu_expert_w4a8(x, w4))
    # a zero residual and an equal down make the two paths identical
    wz = dict(w, gate_rq=np.zeros_like(w["gate_rq"]), up_rq=np.zeros_like(w["up_rq"]),
              down_hq=w["down_lq"], down_hs=w["down_ls"])
    np.testing.assert_array_equal(O.swiglu_expert_split(x, wz, True), low)
    dense = O.swiglu_expert(x, gate, up, down)
    high = O.swiglu_expert_split(x, w, critical=True)
    r = lambda a: np.linalg.norm(a - dense) / np.linalg.norm(dense)
    assert r(high) < r(low) / 2


# ----------------------------------------------------------- miss prefetch ---
def test_prefetch_count_by_hand():
    # 1000 us at 50 GB/s moves 50 MB: five 9.437184 MB experts, capped by 3 free slots
    w = O.prefetch_window(t_remain_us=300.0, t_attn_us=750.0, t_launch_us=50.0)
    assert w == 1000.0
    assert O.prefetch_count(w, 50.0, 9437184, 8) == 5
    assert O.prefetch_count(w, 50.0, 9437184, 3) == 3
    assert O.prefetch_count(w, 50.0, 10_000_000, 8) == 5   # exactly 5.0 experts
    assert O.prefetch_count(w, 50.0, 10_000_001, 8) == 4
    assert O.prefetch_count(0.0, 50.0, 1, 8) == 0
    assert O.prefetch_count(O.prefetch_window(10.0, 0.0, 20.0), 50.0, 1, 8) == 0  # negative window


def test_prefetch_candidates_by_hand():
    lut_row = np.array([0, -1, -1, 3, -1, -1])
    scores = np.array([0.9, 0.1, 0.3, 0.8, 0.3, 0.05], np.float32)
    # predicted set {0, 1, 2, 3, 4}; resident 0 and 3; the rest by score, tie 2/4 to the lower id
    assert O.prefetch_candidates([[0, 2], [4, 1], [3, 2]], scores, lut_row) == [2, 4, 1]


def test_planner_prefetch_hand_trace():
    # 4 slots, 2 layers of 6 experts. Slots 0, 1 hold layer 0's experts 0, 1; slots 2, 3 hold
    # layer 1's experts 2 and 5.
    p = O.LruSlotPlanner(4, 2, 6, residency=[(0, 0), (0, 1), (1, 2), (1, 5)])
    p.plan(0, [0, 1])  # the current step (layer 0) uses slots 0 and 1 at clock 1
    scores = np.array([0.0, 0.0, 0.3, 0.5, 0.2, 0.0], np.float32)
    # layer 1 predicted {2, 3, 4}: 2 is resident; candidates 3 (0.5), 4 (0.2). Free slots: not
    # used at clock 1 and not holding a predicted expert of layer 1: slot 3 only.
    got = p.prefetch(1, [[2, 3], [3, 4]], scores, window_us=1000.0, bw_gbs=50.0, expert_bytes=1000)
    assert got == [(3, 3)]
    assert p.lut[1].tolist() == [-1, -1, 2, 3, -1, -1] and p.owner[3] == (1, 3)
    assert p.last_use == [1, 1, 0, 1]
    # a window that hides nothing prefetches nothing
    q = O.LruSlotPlanner(4, 2, 6, residency=[(0, 0), (0, 1), None, (1, 5)])
    q.plan(0, [0, 1])
    assert q.prefetch(1, [[2, 3]], scores, 0.0, 50.0, 1000) == []
    # an empty slot comes first, then the least recently used free slot
    assert q.prefetch(1, [[2, 3]], scores, 1000.0, 50.0, 1000) == [(3, 2), (2, 3)]
