"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and its host-only logic (slot layout, packing, LRU plan) behaves as defined.

No kernel is launched here. The LRU plan is compared with the oracle's
planner on random traces (bit-exact tables, fills and waves).
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import workloads as W


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_offload.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    names = B.header_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "slot_fill"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version(lib):
    assert "gfx950" in B.moe_version()


@pytest.mark.parametrize("H,F,fmt,expect", [
    (256, 512, B.MOE_F32, (3 * 256 * 512 * 4)),
    (4096, 14336, B.MOE_BF16, 352_321_536),
    (2048, 768, B.MOE_BF16, 3 * 2048 * 768 * 2),
    (7168, 2048, B.MOE_INT4G128, 3 * 7168 * 2048 // 2 + 3 * 7168 * 2048 // 128 * 2),
])
def test_slot_layout_sizes(lib, H, F, fmt, expect):
    lay = B.moe_slot_layout(H, F, fmt)
    assert lay["slot_bytes"] % 4096 == 0
    assert expect <= lay["slot_bytes"] < expect + 4096 + 3 * 256
    for key in ("off_w13", "off_w2", "off_s13", "off_s2"):
        assert lay[key] % 256 == 0


def test_slot_layout_rejects_bad_sizes(lib):
    with pytest.raises(B.MoeError):
        B.moe_slot_layout(100, 512, B.MOE_BF16)
    with pytest.raises(B.MoeError):
        B.moe_slot_layout(7168 + 16, 2048, B.MOE_INT4G128)
    with pytest.raises(B.MoeError):
        B.moe_slot_layout(256, 256, 7)


def _untile_bf16(buf, R, K):
    """Inverse of the documented tile-major bf16 layout: [R, K] from slot bytes."""
    t = buf.view(torch.int16).numpy().reshape(R // 32, K // 16, 2, 32, 8)  # rb, ks, half, row, elem
    return torch.from_numpy(np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4).reshape(R, K))).view(torch.bfloat16)


def test_pack_f32_row_major_interleaved(lib):
    sh = W.reduced(W.shape_of("tiny_e8k2_h256_f512_fp32"), H=64, F=32)
    w = W.expert_weights(sh, 2)
    lay = B.moe_slot_layout(64, 32, B.MOE_F32)
    dst = torch.zeros(lay["slot_bytes"], dtype=torch.uint8)
    B.moe_pack_expert_host(dict(w), 64, 32, B.MOE_F32, dst)
    w13 = dst[:2 * 32 * 64 * 4].view(torch.float32).view(64, 64)
    assert torch.equal(w13[0::2], w["gate"]) and torch.equal(w13[1::2], w["up"])
    assert torch.equal(dst[lay["off_w2"]:lay["off_w2"] + 64 * 32 * 4].view(torch.float32).view(64, 32), w["down"])


def test_pack_bf16_tile_major(lib):
    sh = W.reduced(W.shape_of("mixtral_e8k2_h4096_f14336_bf16"), H=64, F=48)
    w = W.expert_weights(sh, 3)
    lay = B.moe_slot_layout(64, 48, B.MOE_BF16)
    dst = torch.zeros(lay["slot_bytes"], dtype=torch.uint8)
    B.moe_pack_expert_host(dict(w), 64, 48, B.MOE_BF16, dst)
    w13 = _untile_bf16(dst[lay["off_w13"]:lay["off_w13"] + 96 * 64 * 2], 96, 64)
    assert torch.equal(w13[0::2], w["gate"]) and torch.equal(w13[1::2], w["up"])
    w2 = _untile_bf16(dst[lay["off_w2"]:lay["off_w2"] + 64 * 48 * 2], 64, 48)
    assert torch.equal(w2, w["down"])
    # one spot check written out by hand: element (r=33, c=21) of W2
    r, c = 33, 21
    chunk = (r // 32) * (48 // 16) + c // 16
    lane = (r % 32) + 32 * ((c % 16) // 8)
    off = lay["off_w2"] + chunk * 1024 + lane * 16 + (c % 8) * 2
    assert dst[off:off + 2].view(torch.bfloat16).item() == w["down"][r, c].item()


def _untile_int4(buf, R, K):
    """Inverse of the documented tile-major int4 layout: signed codes [R, K]."""
    b = buf.numpy().reshape(R // 32, K // 64, 2, 32, 2, 2, 4)  # rb, kc, khalf, row, h, word, byte
    lo, hi = (b & 0xF).astype(np.int64), (b >> 4).astype(np.int64)
    codes = np.empty((R // 32, K // 64, 2, 32, 2, 2, 8), np.int64)
    codes[..., :4], codes[..., 4:] = lo, hi
    # k = kc*64 + h*32 + khalf*16 + word*8 + i
    codes = codes.transpose(0, 3, 1, 4, 2, 5, 6).reshape(R, K)
    return np.where(codes >= 8, codes - 16, codes)


def test_pack_int4_tile_major_and_scales(lib):
    sh = W.reduced(W.shape_of("dsv3_e256k8s1_h7168_f2048_int4"), H=256, F=128)
    w = W.expert_weights(sh, 1)
    lay = B.moe_slot_layout(256, 128, B.MOE_INT4G128)
    dst = torch.zeros(lay["slot_bytes"], dtype=torch.uint8)
    B.moe_pack_expert_host(dict(w), 256, 128, B.MOE_INT4G128, dst)
    codes = _untile_int4(dst[lay["off_w13"]:lay["off_w13"] + 256 * 128], 256, 256)
    assert np.array_equal(codes[0::2], O.decode_int4(w["gate_q"]))
    assert np.array_equal(codes[1::2], O.decode_int4(w["up_q"]))
    down = _untile_int4(dst[lay["off_w2"]:lay["off_w2"] + 256 * 64], 256, 128)
    assert np.array_equal(down, O.decode_int4(w["down_q"]))
    s13 = dst[lay["off_s13"]:lay["off_s13"] + 256 * 2 * 2].view(torch.bfloat16).view(256, 2)
    assert torch.equal(s13[0::2], w["gate_s"]) and torch.equal(s13[1::2], w["up_s"])
    s2 = dst[lay["off_s2"]:lay["off_s2"] + 256 * 1 * 2].view(torch.bfloat16).view(256, 1)
    assert torch.equal(s2, w["down_s"])


def _lib_state(S, L, E, residency):
    lut = np.full(L * E, -1, np.int32)
    owner = np.full(S, -1, np.int32)
    for s, o in enumerate(residency):
        if o is not None:
            lut[o[0] * E + o[1]] = s
            owner[s] = o[0] * E + o[1]
    return lut, owner, np.zeros(S, np.int64), np.zeros(1, np.int64)


@pytest.mark.parametrize("S,L,E,kmax,seed", [(4, 1, 8, 2, 0), (3, 2, 6, 4, 1), (16, 1, 64, 6, 2),
                                             (7, 3, 10, 3, 3), (1, 1, 5, 2, 4), (300, 6, 128, 8, 5)])
def test_plan_fills_matches_oracle_planner(lib, S, L, E, kmax, seed):
    rng = np.random.default_rng(seed)
    init = [(int(rng.integers(L)), int(e)) for e in rng.choice(E, size=min(S, E) - 1, replace=False)]
    init = list(dict.fromkeys(init)) + [None]
    residency = (init + [None] * S)[:S]
    ref = O.LruSlotPlanner(S, L, E, residency)
    lut, owner, last_use, clock = _lib_state(S, L, E, residency)
    for step in range(200):
        layer = int(rng.integers(L))
        U = sorted({int(e) for e in rng.choice(E, size=int(rng.integers(1, kmax * 3 + 1)))})
        waves = ref.plan(layer, U)
        got = B.moe_plan_fills(lut, owner, last_use, clock, S, L, E, layer, np.array(U))
        assert got["n_waves"] == len(waves)
        exp_fills = [(e, s, wi) for wi, wv in enumerate(waves) for e, s in wv.fills]
        assert list(zip(got["fill_expert"], got["fill_slot"], got["fill_wave"])) == exp_fills
        exp_wave = np.full(E, -1)
        for wi, wv in enumerate(waves):
            exp_wave[wv.compute] = wi
        assert got["wave_of"].tolist() == exp_wave.tolist()
        assert lut.reshape(L, E).tolist() == ref.lut.tolist()
        assert owner.tolist() == [-1 if o is None else o[0] * E + o[1] for o in ref.owner]
        assert last_use.tolist() == ref.last_use and int(clock[0]) == ref.clock


def test_plan_fills_rejects_unsorted_or_out_of_range(lib):
    lut, owner, last_use, clock = _lib_state(2, 1, 4, [None, None])
    for bad in ([2, 1], [0, 4], [-1], [1, 1]):
        with pytest.raises(B.MoeError):
            B.moe_plan_fills(lut, owner, last_use, clock, 2, 1, 4, 0, np.array(bad))
    assert lut.tolist() == [-1] * 4 and int(clock[0]) == 0


def _policy_pair(kind, L, E, rng):
    W = int(rng.integers(1, 6))
    if kind == "mrs":
        return O.MinusRecentScore(L, E, W), B.EvictionPolicy(B.MOE_POLICY_MRS, L, E, W)
    w = [float(v) for v in rng.choice([0.0, 0.25, 0.5, 1.0, 2.0, 3.0], size=4)]
    lam = float(rng.choice([0.0, 0.5, 0.9, 0.95, 1.0]))
    return (O.RoutingHistoryScore(L, E, W, weights=w, lam=lam),
            B.EvictionPolicy(B.MOE_POLICY_HISTORY, L, E, W, params=w + [lam]))


@pytest.mark.parametrize("kind", ["mrs", "history"])
@pytest.mark.parametrize("S,L,E,kmax,seed", [(4, 1, 8, 2, 0), (3, 2, 6, 4, 1), (16, 1, 64, 6, 2),
                                             (7, 3, 10, 3, 3), (1, 1, 5, 2, 4), (40, 4, 32, 6, 5)])
def test_policy_plans_match_oracle(lib, kind, S, L, E, kmax, seed):
    rng = np.random.default_rng(100 + seed)
    init = [(int(rng.integers(L)), int(e)) for e in rng.choice(E, size=min(S, E) - 1, replace=False)]
    residency = (list(dict.fromkeys(init)) + [None] * S)[:S]
    pol_ref, pol = _policy_pair(kind, L, E, rng)
    ref = O.ScoredSlotPlanner(S, L, E, pol_ref, residency)
    lut, owner, last_use, clock = _lib_state(S, L, E, residency)
    for step in range(150):
        layer = int(rng.integers(L))
        logits = rng.normal(size=(int(rng.integers(1, 4)), E)) * 2.0
        if step % 7 == 0:
            logits[:, :E // 2] = logits[:, :1]  # ties in the scores
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :int(rng.integers(1, kmax + 1))]
        U = sorted({int(e) for e in ids.ravel()})
        scores = O.step_scores(logits).astype(np.float32)
        waves = ref.plan(layer, U, scores)
        pol.observe(layer, scores, np.array(U))
        got = pol.plan(lut, owner, last_use, clock, S, layer, np.array(U))
        exp_fills = [(e, s, wi) for wi, wv in enumerate(waves) for e, s in wv.fills]
        assert list(zip(got["fill_expert"], got["fill_slot"], got["fill_wave"])) == exp_fills, step
        assert got["n_waves"] == len(waves)
        assert lut.reshape(L, E).tolist() == ref.lut.tolist()
        assert last_use.tolist() == ref.last_use and int(clock[0]) == ref.clock


def test_policy_lru_kind_equals_plain_plan(lib):
    rng = np.random.default_rng(7)
    S, L, E = 5, 2, 12
    a = _lib_state(S, L, E, [None] * S)
    b = _lib_state(S, L, E, [None] * S)
    pol = B.EvictionPolicy(B.MOE_POLICY_LRU, L, E)
    for step in range(100):
        layer = step % L
        U = np.array(sorted({int(e) for e in rng.choice(E, size=4)}))
        ga = B.moe_plan_fills(*a, S, L, E, layer, U)
        pol.observe(layer, np.zeros(E, np.float32), U)
        gb = pol.plan(*b, S, layer, U)
        assert ga["fill_slot"].tolist() == gb["fill_slot"].tolist()
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_policy_rejects_bad_parameters(lib):
    with pytest.raises(B.MoeError):
        B.EvictionPolicy(B.MOE_POLICY_MRS, 1, 4, 0)
    pol = B.EvictionPolicy(B.MOE_POLICY_HISTORY, 1, 4, 2, params=[1.0, -1.0, 0.0, 0.0, 0.5])
    with pytest.raises(B.MoeError):
        pol.observe(0, np.zeros(4, np.float32), np.array([1]))
    pol = B.EvictionPolicy(B.MOE_POLICY_HISTORY, 1, 4, 2, params=[1.0, 1.0, 0.0, 0.0, 1.5])
    with pytest.raises(B.MoeError):
        pol.observe(0, np.zeros(4, np.float32), np.array([1]))
    pol = B.EvictionPolicy(B.MOE_POLICY_MRS, 1, 4, 2)
    with pytest.raises(B.MoeError):
        pol.observe(0, np.zeros(4, np.float32), np.array([4]))
    assert not pol.state.any()


def test_slot_layout_resplit_extends_int4(lib):
    H, F = 7168, 2048
    base = B.moe_slot_layout(H, F, B.MOE_INT4G128)
    lay = B.moe_slot_layout(H, F, B.MOE_INT4G128_RESPLIT)
    ext = B.moe_slot_layout_resplit(H, F)
    for key in ("off_w13", "off_w2", "off_s13", "off_s2"):
        assert lay[key] == base[key]
    # sections in order, aligned, each large enough for what it holds
    sizes = [("off_s2", H * (F // 128) * 2), ("off_r13", 2 * F * H // 2),
             ("off_rs13", 2 * F * (H // 128) * 2), ("off_h2", H * F), ("off_hs2", H * (F // 128) * 2)]
    offs = {**lay, **ext}
    for (a, size), (b, _) in zip(sizes, sizes[1:]):
        assert offs[b] % 256 == 0 and offs[b] >= offs[a] + size
    assert lay["slot_bytes"] % 4096 == 0 and lay["slot_bytes"] >= offs["off_hs2"] + H * (F // 128) * 2
    with pytest.raises(B.MoeError):
        B.moe_slot_layout_resplit(256 + 64, 256)


def test_quantize_resplit_rejects_bad_sizes(lib):
    w = torch.zeros(64, 192)
    dst = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(B.MoeError):  # H = 192 is not a multiple of 128
        B.moe_quantize_resplit_host(w, w, w.t().contiguous(), 192, 64, dst)
    with pytest.raises(ValueError):  # shapes that do not match H, F
        B.moe_quantize_resplit_host(w, w, w, 192, 64, dst)


def _untile_int8(buf, R, K):
    """Inverse of the documented tile-major 8-bit layout: signed codes [R, K]."""
    b = buf.view(torch.int8).numpy().reshape(R // 32, K // 32, 2, 32, 16)  # rb, kc, khalf, row, byte
    return b.transpose(0, 3, 1, 2, 4).reshape(R, K).astype(np.int64)


def _resplit_inputs(H, F, seed):
    """float32 expert weights with the cases the quantiser must decide alike: an
    all-zero group (scale 0), a lone outlier, and values at exact half steps."""
    g = torch.Generator().manual_seed(seed)
    gate = torch.randn(F, H, generator=g) * 0.02
    up = torch.randn(F, H, generator=g) * 0.02
    down = torch.randn(H, F, generator=g) * 0.02
    gate[0, :128] = 0.0
    up[1, 128:256] = 0.0
    gate[2, 5] = 1.5
    down[3, 7] = -0.75
    # a group whose scale is 2^-6 exactly (max 7 * 2^-6) holding 2.5 and -3.5 steps
    gate[4, :128] = 0.0
    gate[4, 0], gate[4, 1], gate[4, 2] = 7 * 2.0 ** -6, 2.5 * 2.0 ** -6, -3.5 * 2.0 ** -6
    return gate, up, down


@pytest.mark.parametrize("H,F,seed", [(256, 256, 0), (384, 128, 1)])
def test_quantize_resplit_matches_oracle(lib, H, F, seed):
    gate, up, down = _resplit_inputs(H, F, seed)
    ref = O.resplit_expert(gate.numpy(), up.numpy(), down.numpy())
    lay = {**B.moe_slot_layout(H, F, B.MOE_INT4G128_RESPLIT), **B.moe_slot_layout_resplit(H, F)}
    dst = torch.zeros(lay["slot_bytes"], dtype=torch.uint8)
    B.moe_quantize_resplit_host(gate, up, down, H, F, dst)

    def sec(key, nbytes):
        return dst[lay[key]:lay[key] + nbytes]

    def scales(key, R, G):
        return sec(key, R * G * 2).view(torch.bfloat16).float().view(R, G).numpy()

    q13 = _untile_int4(sec("off_w13", 2 * F * H // 2), 2 * F, H)
    r13 = _untile_int4(sec("off_r13", 2 * F * H // 2), 2 * F, H)
    s13, rs13 = scales("off_s13", 2 * F, H // 128), scales("off_rs13", 2 * F, H // 128)
    for j, name in enumerate(("gate", "up")):
        assert np.array_equal(q13[j::2], ref[name + "_q"])
        assert np.array_equal(r13[j::2], ref[name + "_rq"])
        assert np.array_equal(s13[j::2], ref[name + "_s"])
        assert np.array_equal(rs13[j::2], ref[name + "_rs"])
    assert np.array_equal(_untile_int4(sec("off_w2", H * F // 2), H, F), ref["down_lq"])
    assert np.array_equal(scales("off_s2", H, F // 128), ref["down_ls"])
    assert np.array_equal(_untile_int8(sec("off_h2", H * F), H, F), ref["down_hq"])
    assert np.array_equal(scales("off_hs2", H, F // 128), ref["down_hs"])
    # the planted cases: zero groups code to 0 with scale 0; half steps round to even
    assert ref["gate_s"][0, 0] == 0 and not ref["gate_q"][0, :128].any()
    assert ref["gate_s"][4, 0] == 2.0 ** -6
    assert list(ref["gate_q"][4, :3]) == [7, 2, -4]


def test_prefetch_count_matches_oracle(lib):
    rng = np.random.default_rng(31)
    for _ in range(500):
        w = float(rng.choice([-10.0, 0.0, rng.uniform(0, 3000)]))
        bw = float(rng.uniform(1, 100))
        eb = int(rng.integers(1, 400_000_000))
        free = int(rng.integers(0, 20))
        assert B.moe_prefetch_count(w, bw, eb, free) == O.prefetch_count(w, bw, eb, free)
    assert B.moe_prefetch_count(1000.0, 50.0, 10_000_000, 8) == 5


@pytest.mark.parametrize("kind", ["lru", "mrs", "history"])
@pytest.mark.parametrize("S,L,E,kmax,seed", [(6, 2, 8, 2, 0), (20, 3, 16, 4, 1), (5, 4, 6, 3, 2)])
def test_plan_prefetch_matches_oracle(lib, kind, S, L, E, kmax, seed):
    """Steps of a stack: each layer's plan, then a prefetch for the next layer from a
    predicted routing (random windows, including ones that hide nothing); the library's
    tables and prefetch choices equal the oracle planner's at every step."""
    rng = np.random.default_rng(300 + seed)
    init = [(int(rng.integers(L)), int(e)) for e in rng.choice(E, size=min(S, E) - 1, replace=False)]
    residency = (list(dict.fromkeys(init)) + [None] * S)[:S]
    if kind == "lru":
        ref, pol = O.LruSlotPlanner(S, L, E, residency), None
    else:
        pol_ref, pol = _policy_pair(kind, L, E, rng)
        ref = O.ScoredSlotPlanner(S, L, E, pol_ref, residency)
    lut, owner, last_use, clock = _lib_state(S, L, E, residency)
    for step in range(120):
        layer, nxt = step % L, (step + 1) % L
        logits = rng.normal(size=(int(rng.integers(1, 4)), E)) * 2.0
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :int(rng.integers(1, kmax + 1))]
        U = sorted({int(e) for e in ids.ravel()})
        scores = O.step_scores(logits).astype(np.float32)
        if kind == "lru":
            ref.plan(layer, U)
            B.moe_plan_fills(lut, owner, last_use, clock, S, L, E, layer, np.array(U))
        else:
            ref.plan(layer, U, scores)
            pol.observe(layer, scores, np.array(U))
            pol.plan(lut, owner, last_use, clock, S, layer, np.array(U))
        plog = rng.normal(size=(int(rng.integers(1, 4)), E)) * 2.0
        if step % 5 == 0:
            plog[:, :E // 2] = plog[:, :1]  # tied predicted scores
        pids = np.argsort(-plog, axis=1, kind="stable")[:, :kmax]
        psc = O.step_scores(plog).astype(np.float32)
        win = float(rng.choice([0.0, 150.0, 1e6]))
        exp = ref.prefetch(nxt, pids, psc, win, 50.0, 9_437_184)
        got = B.moe_plan_prefetch(pol, lut, owner, last_use, clock, S, L, E, nxt, pids, psc, win,
                                  50.0, 9_437_184)
        assert got == exp, step
        assert lut.reshape(L, E).tolist() == ref.lut.tolist()
        assert last_use.tolist() == ref.last_use and int(clock[0]) == ref.clock
        assert owner.tolist() == [-1 if o is None else o[0] * E + o[1] for o in ref.owner]
