"""int8 activation codes of the int4 expert FFN (the W4A8 row quantisation), bit for bit.

The codes and scales are integer decisions taken in fp32 on both sides, so they
must equal the oracle's quantize_rows_int8 exactly:
  * moe_quantize_rows_int8 on bf16 token rows and fp32 rows (half steps, zero rows);
  * the codes moe_expert_ffn leaves in its workspace (MFMA tiles and the MFMA GEMV):
    the tokens' against the oracle on the same tokens, the SwiGLU intermediate's
    against the oracle on the kernel's own fp32 intermediate (stage parity);
  * a hand-built expert whose output is its h codes times their scale
    (tests/hand_cases.py) on all three int4 paths, including the one-token GEMV that
    quantises inside LDS: the output must equal the hand-worked values exactly.
"""
import numpy as np
import pytest
import torch

import hand_cases as HC
import oracle as O
from expert_offload_routed_amd import binding as B
from expert_offload_routed_amd import harness as Hn
from expert_offload_routed_amd import workloads as W
from gpu_common import say

pytestmark = pytest.mark.gpu

DSV3 = W.shape_of("dsv3_e256k8s1_h7168_f2048_int4")


def _rows_with_edges(R, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(R, K, generator=g) * torch.logspace(-3, 2, R)[:, None]
    a[1] = 0.0                                     # zero row: s = 1, codes 0
    a[2, :8] = torch.tensor([254.0, 5.0, 3.0, -5.0, 1.0, -3.0, 7.0, -7.0])  # s = 2, half steps
    a[2, 8:] = 0.0
    a[3] = -a[0]                                   # sign symmetry
    return a.to(dtype)


@pytest.mark.parametrize("R,K,dtype", [(9, 7168, torch.bfloat16), (6, 2048, torch.float32),
                                       (5, 264, torch.bfloat16), (300, 1408, torch.float32)])
def test_quantize_rows_stage(R, K, dtype):
    a = _rows_with_edges(R, K, dtype, R + K)
    q, s = B.moe_quantize_rows_int8(a.to("cuda"))
    torch.cuda.synchronize()
    qr, sr = O.quantize_rows_int8(a)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert q.cpu().numpy()[2, :8].tolist() == [127, 2, 2, -2, 0, -2, 4, -4]


def test_quantize_rows_rejects_bad_sizes():
    a = torch.zeros(3, 100, device="cuda")
    with pytest.raises(B.MoeError):
        B.moe_quantize_rows_int8(a)  # K % 8 != 0


def _ffn_call(x, ids, E, pool, stride, lut, H, F):
    T, k = ids.shape
    p = B.moe_permute(ids, E)
    wcode = B.MOE_INT4G128
    ws = torch.zeros(B.moe_ffn_workspace_bytes(T, H, F, E, k, wcode), dtype=torch.uint8, device="cuda")
    y = torch.zeros(T * k, H, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_expert_ffn(x, p["perm"], p["offsets"], lut, None, pool, stride, wcode, T, H, F, E, k, y, err, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    return y, ws, p


def _ws_view(ws, off, n, dtype):
    nbytes = n * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).cpu().numpy()


@pytest.mark.parametrize("T", [8, 40])  # MFMA GEMV (groups of 2-32 rows), MFMA tiles
def test_ffn_workspace_codes_full_size(T):
    shape = W.reduced(DSV3, E=12, k=8, H=7168, F=2048)
    E, k, H, F = shape.E, shape.k, shape.H, shape.F
    say(f"workspace codes {shape.name} T={T}")
    store = Hn.ExpertStore(shape)
    pool = torch.empty(E * store.stride, dtype=torch.uint8, device="cuda")
    for e in range(E):
        pool[e * store.stride:(e + 1) * store.stride].copy_(store.host[W.blob_of(shape, 0, e)])
    lut = torch.arange(E, dtype=torch.int32, device="cuda")
    x = W.tokens(shape, T, device="cuda")
    wr, b = W.router(shape, device="cuda")
    _, ids, _ = B.moe_route(x, wr, b, k)
    y, ws, p = _ffn_call(x, ids, E, pool, store.stride, lut, H, F)
    o = B.moe_ffn_workspace_offsets(T, H, F, E, k, B.MOE_INT4G128)
    xq, xs = _ws_view(ws, o["xq"], T * H, torch.int8), _ws_view(ws, o["xs"], T, torch.float32)
    qr, sr = O.quantize_rows_int8(x)
    assert np.array_equal(xq.reshape(T, H), qr)
    assert np.array_equal(xs.view(np.uint32), sr.view(np.uint32))
    h = _ws_view(ws, o["h"], T * k * F, torch.float32).reshape(T * k, F)
    hq, hs = _ws_view(ws, o["hq"], T * k * F, torch.int8), _ws_view(ws, o["hs"], T * k, torch.float32)
    qh, sh = O.quantize_rows_int8(h)  # on the kernel's own fp32 intermediate
    assert np.array_equal(hq.reshape(T * k, F), qh)
    assert np.array_equal(hs.view(np.uint32), sh.view(np.uint32))
    say(f"  {T * H} token codes and {T * k * F} intermediate codes equal")


@pytest.mark.parametrize("T", [1, 2, 8, 33, 40])  # one-token GEMV (LDS codes), MFMA GEMV, MFMA tiles
def test_ffn_hand_expert_exposes_codes(T):
    H, F, E = 512, 256, 4
    say(f"hand expert T={T}")
    w = HC.w4a8_expert(H, F)
    lay = B.moe_slot_layout(H, F, B.MOE_INT4G128)
    stride = lay["slot_bytes"]
    host = torch.zeros(stride, dtype=torch.uint8, pin_memory=True)
    B.moe_pack_expert_host(dict(w), H, F, B.MOE_INT4G128, host)
    pool = host.to("cuda")
    lut = torch.tensor([-1, -1, 0, -1], dtype=torch.int32, device="cuda")  # expert 2 in slot 0
    x = torch.from_numpy(HC.tokens(T, H)).to(torch.bfloat16).to("cuda")
    ids = torch.full((T, 1), 2, dtype=torch.int32, device="cuda")
    y, ws, p = _ffn_call(x, ids, E, pool, stride, lut, H, F)
    got = y.cpu().numpy().astype(np.float64)  # sorted position t = token t (one expert)
    assert got.tolist() == HC.expected_y(T, H, F).tolist()
    if T >= 2:  # these paths leave the codes in the workspace
        o = B.moe_ffn_workspace_offsets(T, H, F, E, 1, B.MOE_INT4G128)
        xq, xs, hq, hs = HC.expected_codes(T, H, F)
        assert np.array_equal(_ws_view(ws, o["xq"], T * H, torch.int8).reshape(T, H), xq)
        assert np.array_equal(_ws_view(ws, o["xs"], T, torch.float32), xs)
        assert np.array_equal(_ws_view(ws, o["hq"], T * F, torch.int8).reshape(T, F), hq)
        assert np.array_equal(_ws_view(ws, o["hs"], T, torch.float32), hs)
