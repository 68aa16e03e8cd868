"""Thin ctypes binding of libmoe_offload (same names as the C ABI in include/moe_offload.h).

Argument marshalling only: tensors become device pointers, streams become HIP
stream handles, missing outputs are allocated with torch, and a non-zero
status raises ``MoeError``. Every step of the layer runs in the library's
kernels; there is no fallback path, and loading fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

from .build import LIB_PATH

MOE_F32, MOE_BF16, MOE_INT4G128, MOE_INT4G128_RESPLIT = 0, 1, 2, 3
MOE_ERR_ABSENT, MOE_ERR_STALE_TAG, MOE_ERR_SYNC = 1, 2, 4
_STATUS = {-1: "invalid argument", -2: "unsupported dtype or shape", -3: "HIP runtime error"}

_vp, _i32, _i64, _u64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t

_SIGNATURES = {
    "moe_route": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_permute": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_permute": (_i32, [_vp, _i32, _vp, _vp] + [_i32] * 5 + [_vp] * 11),
    "moe_slot_layout": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_pack_expert_host": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "moe_slot_layout_resplit": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_quantize_resplit_host": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp]),
    "moe_critical_split": (_i32, [_vp, _i32, ctypes.c_float, _vp, _i32, _vp, _vp]),
    "moe_step_scores": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "moe_ffn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_ffn_workspace_offsets": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "moe_expert_ffn_noalloc": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_noalloc_scratch_bytes": (_sz, []),
    "moe_quantize_rows_int8": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_expert_ffn": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _i32, _i32, _i32, _i32, _i32,
                              _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_combine": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _vp]),
    "slot_fill": (_i32, [_vp, _sz, _i32, _vp, _sz, _vp, _i32, _vp, _vp, _u64, _vp, _vp, _vp]),
    "slot_commit": (_i32, [_vp, _i32, _vp, _i32, _vp, _u64, _vp, _vp]),
    "slot_prefetch": (_i32, [_vp, _sz, _i32, _vp, _sz, _vp, _u64, _vp]),
    "moe_plan_fills": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp]),
    "moe_policy_state_doubles": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_policy_observe": (_i32, [_i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "moe_plan_fills_policy": (_i32, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_prefetch_count": (_i32, [ctypes.c_double, ctypes.c_double, _sz, _i32]),
    "moe_plan_prefetch": (_i32, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _vp, _i32, _vp, ctypes.c_double, ctypes.c_double, _sz, _vp, _vp,
                                 _vp]),
    "moe_ctx_workspace_bytes": (_sz, [_i32] * 9),
    "moe_ctx_create": (_i32, [ctypes.POINTER(_vp)] + [_i32] * 10 + [_vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp,
                                                                   _vp, _vp, _sz, _vp, _vp]),
    "moe_ctx_destroy": (_i32, [_vp]),
    "moe_ctx_place": (_i32, [_vp, _i32, _i32, _i32]),
    "moe_layer_forward": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp]),
    "moe_ctx_forward_steps": (_i32, [_vp, _i32, _vp, ctypes.POINTER(_vp), _i32, ctypes.POINTER(_vp),
                                     ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32]),
    "moe_ctx_read_tables": (_i32, [_vp, _vp, _vp, _vp, _vp]),
    "moe_ctx_outputs": (_i32, [_vp] + [ctypes.POINTER(_vp)] * 6),
    "moe_ctx_set_timing": (_i32, [_vp, _i32]),
    "moe_ctx_set_prefetch": (_i32, [_vp, _i32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double]),
    "moe_ctx_prefetch_counters": (_i32, [_vp, _vp]),
    "moe_ctx_set_policy": (_i32, [_vp, _i32, _i32, _vp]),
    "moe_ctx_set_orchestration": (_i32, [_vp, _i32]),
    "moe_ctx_step_scores": (_i32, [_vp, _vp]),
    "moe_ctx_set_split": (_i32, [_vp, _i32, ctypes.c_float, _vp, ctypes.c_float]),
    "moe_ctx_set_staging": (_i32, [_vp, _i32, _i32, _i32]),
    "moe_ctx_stage_counters": (_i32, [_vp, _vp]),
    "moe_ctx_counters": (_i32, [_vp, _vp]),
    "moe_ctx_ffn_time": (_i32, [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_long)]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} failed: {rc} ({_STATUS.get(rc, 'unknown status')})")
        self.rc = rc


_LIB: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` "
                               "or expert_offload_routed_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            if hasattr(handle, name):
                fn = getattr(handle, name)
                fn.restype, fn.argtypes = res, args
        _LIB = handle
    return _LIB


def header_functions() -> list[str]:
    """Names of the functions declared in include/*.h."""
    inc = os.path.join(os.path.dirname(os.path.dirname(LIB_PATH)), "include")
    names = []
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            names += re.findall(r"^(?:const\s+)?\w+\s*\*?\s+(\w+)\s*\(", src, flags=re.M)
    return names


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MoeError(name, rc)


# ------------------------------------------------------------- marshalling --
def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _host(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("expected a contiguous array")
        return a.ctypes.data
    if a.is_cuda or not a.is_contiguous():
        raise ValueError("expected a contiguous host tensor")
    return a.data_ptr()


def _stream(s) -> int:
    if s is None:
        s = torch.cuda.current_stream()
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


# ----------------------------------------------------------------- gating --
def moe_route(x, w_router, bias, k: int, renorm: bool = True, logits=None, topk_ids=None,
              topk_w=None, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty(T, E, device=dev, dtype=torch.float32) if logits is None else logits
    topk_ids = torch.empty(T, k, device=dev, dtype=torch.int32) if topk_ids is None else topk_ids
    topk_w = torch.empty(T, k, device=dev, dtype=torch.float32) if topk_w is None else topk_w
    if tuple(w_router.shape) != (E, H) or (bias is not None and bias.numel() != E):
        raise ValueError("moe_route: w_router must be [E, H] and bias [E]")
    if logits.numel() < T * E or topk_ids.numel() < T * k or topk_w.numel() < T * k:
        raise ValueError("moe_route: output buffers too small")
    if w_router.dtype != x.dtype:
        raise TypeError("x and w_router must share a dtype")
    _call("moe_route", _dev(x), dtype_code(x), _dev(w_router), _dev(bias), T, H, E, k, int(renorm),
          _dev(logits), _dev(topk_ids), _dev(topk_w), _stream(stream))
    return logits, topk_ids, topk_w


def moe_permute(topk_ids, E: int, out: dict | None = None, stream=None) -> dict:
    T, k = topk_ids.shape
    dev = topk_ids.device
    o = out or {}
    o.setdefault("counts", torch.empty(E, device=dev, dtype=torch.int32))
    o.setdefault("offsets", torch.empty(E + 1, device=dev, dtype=torch.int32))
    o.setdefault("perm", torch.empty(max(T * k, 1), device=dev, dtype=torch.int32))
    o.setdefault("inv", torch.empty(max(T * k, 1), device=dev, dtype=torch.int32))
    o.setdefault("distinct", torch.empty(E, device=dev, dtype=torch.int32))
    o.setdefault("n_distinct", torch.empty(1, device=dev, dtype=torch.int32))
    need = {"counts": E, "offsets": E + 1, "perm": T * k, "inv": T * k, "distinct": E, "n_distinct": 1}
    for name, n in need.items():
        if o[name].numel() < n or o[name].dtype != torch.int32:
            raise ValueError(f"moe_permute: output '{name}' needs {n} int32 elements")
    _call("moe_permute", _dev(topk_ids), T, k, E, _dev(o["counts"]), _dev(o["offsets"]),
          _dev(o["perm"]), _dev(o["inv"]), _dev(o["distinct"]), _dev(o["n_distinct"]),
          _stream(stream))
    return o


def moe_route_permute(x, w_router, bias, k: int, renorm: bool = True, sync_counter=None, stream=None):
    """Route and permute in one call; returns (logits, ids, weights, permutation dict)."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty(T, E, device=dev, dtype=torch.float32)
    ids = torch.empty(T, k, device=dev, dtype=torch.int32)
    w = torch.empty(T, k, device=dev, dtype=torch.float32)
    o = {n: torch.empty(c, device=dev, dtype=torch.int32) for n, c in (
        ("counts", E), ("offsets", E + 1), ("perm", max(T * k, 1)), ("inv", max(T * k, 1)),
        ("distinct", E), ("n_distinct", 1))}
    if sync_counter is None:
        sync_counter = torch.zeros(1, device=dev, dtype=torch.int32)
    if w_router.dtype != x.dtype or tuple(w_router.shape) != (E, H):
        raise ValueError("moe_route_permute: w_router must be [E, H] in the dtype of x")
    _call("moe_route_permute", _dev(x), dtype_code(x), _dev(w_router), _dev(bias), T, H, E, k,
          int(renorm), _dev(logits), _dev(ids), _dev(w), _dev(o["counts"]), _dev(o["offsets"]),
          _dev(o["perm"]), _dev(o["inv"]), _dev(o["distinct"]), _dev(o["n_distinct"]),
          _dev(sync_counter), _stream(stream))
    return logits, ids, w, o


# ------------------------------------------------------------ slot layout --
def moe_slot_layout(H: int, F: int, w_dtype: int) -> dict:
    vals = [ctypes.c_size_t() for _ in range(5)]
    _call("moe_slot_layout", H, F, w_dtype, *[ctypes.addressof(v) for v in vals])
    return dict(zip(("slot_bytes", "off_w13", "off_w2", "off_s13", "off_s2"), (v.value for v in vals)))


def moe_slot_layout_resplit(H: int, F: int) -> dict:
    vals = [ctypes.c_size_t() for _ in range(4)]
    _call("moe_slot_layout_resplit", H, F, *[ctypes.addressof(v) for v in vals])
    return dict(zip(("off_r13", "off_rs13", "off_h2", "off_hs2"), (v.value for v in vals)))


def moe_quantize_resplit_host(gate, up, down, H: int, F: int, dst) -> None:
    """Quantise one expert from float32 host tensors (nn.Linear orientation) into a
    MOE_INT4G128_RESPLIT slot image dst (host uint8, slot bytes)."""
    ts = [t.detach().to("cpu", torch.float32).contiguous() for t in (gate, up, down)]
    if (tuple(ts[0].shape) != (F, H) or tuple(ts[1].shape) != (F, H)
            or tuple(ts[2].shape) != (H, F)):
        raise ValueError("moe_quantize_resplit_host: gate, up must be [F, H] and down [H, F]")
    _call("moe_quantize_resplit_host", *[_host(t) for t in ts], H, F, _host(dst))


def moe_step_scores(logits, T: int, E: int, scores=None, stream=None):
    if scores is None:
        scores = torch.empty(E, device=logits.device, dtype=torch.float32)
    if logits.numel() < T * E or scores.numel() < E:
        raise ValueError("moe_step_scores: an argument is smaller than its shape needs")
    _call("moe_step_scores", _dev(logits), T, E, _dev(scores), _stream(stream))
    return scores


def moe_critical_split(scores, E: int, threshold: float, mask_in=None, rows: int = 1,
                       mask_out=None, stream=None):
    if mask_out is None:
        mask_out = torch.empty(rows, E, device=scores.device, dtype=torch.int32)
    if (scores.numel() < E or mask_out.numel() < rows * E
            or (mask_in is not None and mask_in.numel() < rows * E)):
        raise ValueError("moe_critical_split: an argument is smaller than its shape needs")
    _call("moe_critical_split", _dev(scores), E, ctypes.c_float(threshold), _dev(mask_in), rows,
          _dev(mask_out), _stream(stream))
    return mask_out


def moe_pack_expert_host(weights: dict, H: int, F: int, w_dtype: int, dst) -> None:
    """Pack one expert (host tensors, nn.Linear orientation) into dst (host uint8, slot bytes)."""
    def h(name):
        t = weights.get(name)
        if t is None:
            return None
        t = t.contiguous()
        weights[name] = t
        return _host(t)
    if w_dtype == MOE_INT4G128:
        args = [h("gate_q"), h("up_q"), h("down_q"), h("gate_s"), h("up_s"), h("down_s")]
    else:
        args = [h("gate"), h("up"), h("down"), None, None, None]
    _call("moe_pack_expert_host", *args, H, F, w_dtype, _host(dst))


# ------------------------------------------------------------- expert FFN --
def moe_ffn_workspace_bytes(T, H, F, E, k, w_dtype) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, H, F, E, k, w_dtype))


def moe_ffn_workspace_offsets(T, H, F, E, k, w_dtype) -> dict:
    offs = (ctypes.c_size_t * 5)()
    _call("moe_ffn_workspace_offsets", T, H, F, E, k, w_dtype, ctypes.cast(offs, _vp))
    return dict(zip(("h", "xq", "xs", "hq", "hs"), (int(v) for v in offs)))


def moe_quantize_rows_int8(a, stream=None):
    """Per-row int8 codes and scales of a [rows, K] fp32 or bf16 device tensor."""
    a = a.contiguous()
    rows, K = a.shape
    q = torch.empty(rows, K, dtype=torch.int8, device=a.device)
    s = torch.empty(rows, dtype=torch.float32, device=a.device)
    _call("moe_quantize_rows_int8", _dev(a), dtype_code(a), rows, K, _dev(q), _dev(s),
          _stream(stream))
    return q, s


def moe_expert_ffn(x, perm, offsets, lut_row, group_mask, pool, slot_stride: int, w_dtype: int,
                   T: int, H: int, F: int, E: int, k: int, y_perm, err_word, workspace, stream=None):
    num_slots = pool.numel() // slot_stride
    if (x.numel() < T * H or perm.numel() < T * k or offsets.numel() < E + 1 or lut_row.numel() < E
            or y_perm.numel() < T * k * H or (group_mask is not None and group_mask.numel() < E)):
        raise ValueError("moe_expert_ffn: an argument is smaller than its shape needs")
    _call("moe_expert_ffn", _dev(x), dtype_code(x), _dev(perm), _dev(offsets), _dev(lut_row),
          _dev(group_mask), _dev(pool), slot_stride, num_slots, w_dtype, T, H, F, E, k, _dev(y_perm),
          _dev(err_word), _dev(workspace), workspace.numel() * workspace.element_size(),
          _stream(stream))


def moe_expert_ffn_noalloc(x, perm, offsets, lut_row, group_mask, pool, slot_stride: int,
                           w_dtype: int, T: int, H: int, F: int, E: int, k: int, y_perm, err_word,
                           stream=None):
    num_slots = pool.numel() // slot_stride
    if (x.numel() < T * H or perm.numel() < T * k or offsets.numel() < E + 1 or lut_row.numel() < E
            or y_perm.numel() < T * k * H or (group_mask is not None and group_mask.numel() < E)):
        raise ValueError("moe_expert_ffn_noalloc: an argument is smaller than its shape needs")
    _call("moe_expert_ffn_noalloc", _dev(x), dtype_code(x), _dev(perm), _dev(offsets), _dev(lut_row),
          _dev(group_mask), _dev(pool), slot_stride, num_slots, w_dtype, T, H, F, E, k, _dev(y_perm),
          _dev(err_word), _stream(stream))


def moe_noalloc_scratch_bytes() -> int:
    return int(lib().moe_noalloc_scratch_bytes())


# ---------------------------------------------------------------- combine --
def moe_combine(y_perm, inv, topk_w, T: int, k: int, H: int, shared_y=None, out=None,
                out_dtype=torch.bfloat16, stream=None):
    if out is None:
        out = torch.empty(T, H, device=topk_w.device, dtype=out_dtype)
    n_sh = 0 if shared_y is None else shared_y.shape[0]
    if (inv.numel() < T * k or topk_w.numel() < T * k or out.numel() < T * H
            or (shared_y is not None and shared_y.numel() < n_sh * T * H)):
        raise ValueError("moe_combine: an argument is smaller than its shape needs")
    _call("moe_combine", _dev(y_perm), _dev(inv), _dev(topk_w), T, k, H, _dev(shared_y), n_sh,
          _dev(out), dtype_code(out), _stream(stream))
    return out


# -------------------------------------------------------------- slot fill --
def slot_fill(pool, slot_stride: int, slot: int, host_src, nbytes: int, lut, lut_index: int, owner,
              slot_tags, tag: int, err_word, fill_stream=None, compute_stream=None):
    src = host_src if isinstance(host_src, int) else host_src.data_ptr()
    _call("slot_fill", _dev(pool), slot_stride, slot, src, nbytes, _dev(lut), lut_index, _dev(owner),
          _dev(slot_tags), tag, _dev(err_word), _stream(fill_stream), _stream(compute_stream))


def slot_prefetch(pool, slot_stride: int, slot: int, host_src, nbytes: int, slot_tags, tag: int,
                  fill_stream=None):
    src = host_src if isinstance(host_src, int) else host_src.data_ptr()
    _call("slot_prefetch", _dev(pool), slot_stride, slot, src, nbytes, _dev(slot_tags), tag,
          _stream(fill_stream))


def slot_commit(lut, lut_index: int, owner, slot: int, slot_tags, tag: int, err_word, stream=None):
    _call("slot_commit", _dev(lut), lut_index, _dev(owner), slot, _dev(slot_tags), tag,
          _dev(err_word), _stream(stream))


# --------------------------------------------------------- host residency --
def moe_plan_fills(lut: np.ndarray, owner: np.ndarray, last_use: np.ndarray, clock: np.ndarray,
                   S: int, L: int, E: int, layer: int, distinct: np.ndarray) -> dict:
    """Run the host LRU plan on numpy state arrays (updated in place)."""
    return _plan(None, lut, owner, last_use, clock, S, L, E, layer, distinct)


def _plan(policy, lut, owner, last_use, clock, S, L, E, layer, distinct) -> dict:
    assert lut.dtype == np.int32 and owner.dtype == np.int32
    assert last_use.dtype == np.int64 and clock.dtype == np.int64
    d = np.ascontiguousarray(distinct, dtype=np.int32)
    n = d.size
    wave_of = np.empty(E, np.int32)
    is_hit = np.empty(E, np.int32)
    fe, fs, fw = (np.empty(max(n, 1), np.int32) for _ in range(3))
    nf, nw = np.zeros(1, np.int32), np.zeros(1, np.int32)
    tail = (_host(lut), _host(owner), _host(last_use), _host(clock), S, L, E, layer,
            _host(d) if n else None, n, _host(wave_of), _host(is_hit), _host(fe), _host(fs), _host(fw),
            _host(nf), _host(nw))
    if policy is None:
        _call("moe_plan_fills", *tail)
    else:
        _call("moe_plan_fills_policy", policy.kind, _host(policy.state), policy.window,
              _host(policy.params) if policy.params is not None else None, *tail)
    k = int(nf[0])
    return dict(wave_of=wave_of, is_hit=is_hit, fill_expert=fe[:k].copy(), fill_slot=fs[:k].copy(),
                fill_wave=fw[:k].copy(), n_waves=int(nw[0]))


MOE_POLICY_LRU, MOE_POLICY_MRS, MOE_POLICY_HISTORY = 0, 1, 2
MOE_ORCH_HOST, MOE_ORCH_DEVICE = 0, 1


def moe_prefetch_count(window_us: float, bw_gbs: float, expert_bytes: int, free_slots: int) -> int:
    return int(lib().moe_prefetch_count(window_us, bw_gbs, expert_bytes, free_slots))


def moe_plan_prefetch(policy, lut, owner, last_use, clock, S: int, L: int, E: int, layer: int,
                      pred_ids, pred_scores, window_us: float, bw_gbs: float,
                      expert_bytes: int) -> list:
    """Host prefetch plan on numpy state arrays (updated in place); policy None = LRU.
    Returns [(expert, slot)]."""
    p = np.ascontiguousarray(np.asarray(pred_ids).ravel(), dtype=np.int32)
    sc = np.ascontiguousarray(pred_scores, dtype=np.float32)
    fe, fs = np.empty(E, np.int32), np.empty(E, np.int32)
    nf = np.zeros(1, np.int32)
    kind = MOE_POLICY_LRU if policy is None else policy.kind
    state = None if policy is None else _host(policy.state)
    window = 1 if policy is None else policy.window
    params = None if policy is None or policy.params is None else _host(policy.params)
    _call("moe_plan_prefetch", kind, state, window, params, _host(lut), _host(owner),
          _host(last_use), _host(clock), S, L, E, layer, _host(p) if p.size else None, p.size,
          _host(sc), window_us, bw_gbs, expert_bytes, _host(fe), _host(fs), _host(nf))
    return [(int(fe[i]), int(fs[i])) for i in range(int(nf[0]))]


class EvictionPolicy:
    """Host state of an eviction policy (moe_policy_* in include/moe_offload.h)."""

    def __init__(self, kind: int, L: int, E: int, window: int = 1, params=None):
        self.kind, self.L, self.E, self.window = kind, L, E, window
        self.params = None if params is None else np.ascontiguousarray(params, dtype=np.float64)
        n = int(lib().moe_policy_state_doubles(kind, L, E, window))
        if kind != MOE_POLICY_LRU and n == 0:
            raise MoeError("moe_policy_state_doubles", -1)
        self.state = np.zeros(max(n, 1), np.float64)

    def observe(self, layer: int, scores: np.ndarray, distinct: np.ndarray) -> None:
        sc = np.ascontiguousarray(scores, dtype=np.float32)
        d = np.ascontiguousarray(distinct, dtype=np.int32)
        _call("moe_policy_observe", self.kind, _host(self.state), self.L, self.E, self.window, layer,
              _host(sc), _host(d) if d.size else None, d.size,
              _host(self.params) if self.params is not None else None)

    def plan(self, lut, owner, last_use, clock, S: int, layer: int, distinct) -> dict:
        return _plan(self, lut, owner, last_use, clock, S, self.L, self.E, layer, distinct)


def moe_version() -> str:
    return lib().moe_version().decode()


# ------------------------------------------------------------ layer runtime --
def moe_ctx_workspace_bytes(t_max, H, F, E, k, L, S, w_dtype, n_shared) -> int:
    return int(lib().moe_ctx_workspace_bytes(t_max, H, F, E, k, L, S, w_dtype, n_shared))


class LayerContext:
    """Handle of a moe_layer_ctx (include/moe_runtime.h); keeps its buffers alive."""

    def __init__(self, *, t_max, H, F, E, k, L, S, x_dtype, w_dtype, n_shared, pool, slot_stride, lut,
                 owner, tags, host_store, blob_of: np.ndarray, shared_pool, err, compute_stream=None,
                 fill_stream=None):
        dev = pool.device
        self.t_max, self.H, self.E, self.k, self.L, self.S = t_max, H, E, k, L, S
        self.pool_slots = pool.numel() // slot_stride
        self.compute_stream = compute_stream or torch.cuda.current_stream(dev)
        self.fill_stream = fill_stream or torch.cuda.Stream(device=dev)
        nbytes = moe_ctx_workspace_bytes(t_max, H, F, E, k, L, S, w_dtype, n_shared)
        if nbytes == 0:
            raise ValueError("moe_ctx_workspace_bytes: bad sizes")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.blob_of = np.ascontiguousarray(blob_of, dtype=np.int32)
        if self.blob_of.size != L * E:
            raise ValueError("blob_of must hold L*E entries")
        if tags.dtype != torch.int64 or tags.numel() < S or owner.numel() < S or lut.numel() < L * E:
            raise ValueError("tables too small")
        if pool.numel() < (S + n_shared) * slot_stride:
            raise ValueError("pool must hold S routed slots followed by n_shared shared slots")
        self._keep = (pool, lut, owner, tags, host_store, shared_pool, err)
        self.handle = _vp()
        _call("moe_ctx_create", ctypes.byref(self.handle), t_max, H, F, E, k, L, S, x_dtype, w_dtype,
              n_shared, _dev(pool), slot_stride, _dev(lut), _dev(owner), _dev(tags), _host(host_store),
              _host(self.blob_of), _dev(shared_pool), _dev(err), _dev(self.ws), nbytes,
              _stream(self.compute_stream), _stream(self.fill_stream))

    def place(self, slot: int, layer: int, expert: int) -> None:
        _call("moe_ctx_place", self.handle, slot, layer, expert)

    def forward(self, layer: int, x, w_router, bias, out, stats: np.ndarray | None = None) -> None:
        T = x.shape[0]
        if T > self.t_max or x.shape[1] != self.H or tuple(w_router.shape) != (self.E, self.H):
            raise ValueError("moe_layer_forward: shape mismatch")
        if out.numel() < T * self.H or (bias is not None and bias.numel() != self.E):
            raise ValueError("moe_layer_forward: output or bias size")
        _call("moe_layer_forward", self.handle, layer, _dev(x), T, _dev(w_router), _dev(bias), _dev(out),
              dtype_code(out), _host(stats))

    def forward_steps(self, steps, out_dtype_code: int) -> None:
        """steps: list of (layer, x, w_router, bias, out), run in order by one moe_ctx_forward_steps call."""
        n = len(steps)
        if n == 0:
            return
        T = steps[0][1].shape[0]
        for layer, x, wr, b, out in steps:
            if (x.shape[0] != T or T > self.t_max or x.shape[1] != self.H or tuple(wr.shape) != (self.E, self.H)
                    or out.numel() < T * self.H or (b is not None and b.numel() != self.E)
                    or not 0 <= layer < self.L):
                raise ValueError("moe_ctx_forward_steps: shape mismatch")
        layers = np.array([s[0] for s in steps], np.int32)
        ptrs = lambda i: (ctypes.c_void_p * n)(*[_dev(s[i]) for s in steps])
        _call("moe_ctx_forward_steps", self.handle, n, _host(layers), ptrs(1), T, ptrs(2), ptrs(3), ptrs(4),
              out_dtype_code)

    def tables(self):
        lut = np.empty(self.L * self.E, np.int32)
        owner = np.empty(self.S, np.int32)
        last = np.empty(self.S, np.int64)
        clock = np.zeros(1, np.int64)
        _call("moe_ctx_read_tables", self.handle, _host(lut), _host(owner), _host(last), _host(clock))
        return lut, owner, last, int(clock[0])

    def outputs(self, T: int) -> dict:
        """Views into the workspace of the last step's routing and permutation."""
        ptrs = [_vp() for _ in range(6)]
        _call("moe_ctx_outputs", self.handle, *[ctypes.byref(p) for p in ptrs])
        base = self.ws.data_ptr()
        E, k = self.E, self.k

        def view(p, n, dtype, shape):
            off = p.value - base
            return self.ws[off:off + n * 4].view(dtype).view(*shape)
        return dict(logits=view(ptrs[0], T * E, torch.float32, (T, E)),
                    ids=view(ptrs[1], T * k, torch.int32, (T, k)),
                    topk_w=view(ptrs[2], T * k, torch.float32, (T, k)),
                    perm=view(ptrs[3], T * k, torch.int32, (T * k,)),
                    offsets=view(ptrs[4], E + 1, torch.int32, (E + 1,)),
                    inv=view(ptrs[5], T * k, torch.int32, (T * k,)))

    def counters(self) -> dict:
        c = np.zeros(4, np.int64)
        _call("moe_ctx_counters", self.handle, _host(c))
        return dict(distinct=int(c[0]), hits=int(c[1]), fills=int(c[2]), waves=int(c[3]))

    def set_prefetch(self, on: bool, t_remain_us: float = 0.0, t_attn_us: float = 0.0,
                     t_launch_us: float = 0.0, bw_gbs: float = 1.0) -> None:
        _call("moe_ctx_set_prefetch", self.handle, int(on), t_remain_us, t_attn_us, t_launch_us, bw_gbs)

    def prefetch_counters(self) -> dict:
        out = np.zeros(2, np.int64)
        _call("moe_ctx_prefetch_counters", self.handle, _host(out))
        return {"prefetched": int(out[0]), "prefetch_used": int(out[1])}

    def set_timing(self, on: bool) -> None:
        _call("moe_ctx_set_timing", self.handle, int(on))

    def set_orchestration(self, mode: int) -> None:
        """MOE_ORCH_HOST or MOE_ORCH_DEVICE (plans and fills on the GPU, no host wait per step)."""
        _call("moe_ctx_set_orchestration", self.handle, mode)

    def set_policy(self, kind: int, window: int = 1, params=None) -> None:
        """Eviction policy of the residency plans (MOE_POLICY_LRU / _MRS / _HISTORY)."""
        p = None if params is None else np.ascontiguousarray(params, dtype=np.float64)
        self._policy_params = p  # kept alive while the call reads it
        _call("moe_ctx_set_policy", self.handle, kind, window, _host(p) if p is not None else None)

    def set_split(self, enable: bool, theta: float = 0.0, beta=None, gamma: float = 1.0) -> None:
        """Split-precision routing over MOE_INT4G128_RESPLIT experts: routed expert e of
        layer l on W^H when its step score >= theta * beta[l] * gamma, else on W^L."""
        b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float32)
        self._split_beta = b
        _call("moe_ctx_set_split", self.handle, int(enable), ctypes.c_float(theta),
              _host(b) if b is not None else None, ctypes.c_float(gamma))

    def set_staging(self, enable: bool, threshold: int = -1) -> None:
        """Prefill full-layer staging in two buffers of E slots after the routed and shared
        slots of the pool (threshold -1: floor(resident slots of the layer / k))."""
        _call("moe_ctx_set_staging", self.handle, int(enable), threshold, self.pool_slots)

    def stage_counters(self) -> dict:
        out = np.zeros(2, np.int64)
        _call("moe_ctx_stage_counters", self.handle, _host(out))
        return {"staged_steps": int(out[0]), "stage_copies": int(out[1])}

    def step_scores(self) -> np.ndarray:
        """Routing scores [E] of the latest step (needs split precision or a policy other
        than LRU)."""
        out = np.zeros(self.E, np.float32)
        _call("moe_ctx_step_scores", self.handle, _host(out))
        return out

    def ffn_time(self) -> tuple[float, int]:
        ms, n = ctypes.c_double(), ctypes.c_long()
        _call("moe_ctx_ffn_time", self.handle, ctypes.byref(ms), ctypes.byref(n))
        return ms.value, n.value

    def close(self) -> None:
        if getattr(self, "handle", None) and self.handle.value:
            lib().moe_ctx_destroy(self.handle)
            self.handle = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
