"""Device state of one routed-expert workload and a layer step over the C ABI.

PyTorch provides device memory, pinned host memory and streams; every step of
the layer is a call into libmoe_offload:

  moe_route -> moe_permute -> (D2H of the distinct routed set, the one host
  synchronisation per layer) -> moe_plan_fills (host LRU plan) ->
  moe_expert_ffn on the resident groups while slot_fill copies the misses on
  the fill stream -> moe_expert_ffn on the filled groups (one pass per wave)
  -> moe_expert_ffn of the shared experts -> moe_combine.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B
from . import workloads as W

WFMT_CODE = {"f32": B.MOE_F32, "bf16": B.MOE_BF16, "int4g128": B.MOE_INT4G128}


def weights_to_host(w: dict) -> dict:
    return {k: v.detach().to("cpu").contiguous() for k, v in w.items()}


class ExpertStore:
    """Pinned host store: one packed expert (slot layout) per weight set."""

    def __init__(self, shape: W.MoEShape, *, shared: bool = False, gen_device="cuda"):
        self.shape = shape
        self.wcode = WFMT_CODE[shape.wfmt]
        self.layout = B.moe_slot_layout(shape.H, shape.F, self.wcode)
        self.stride = self.layout["slot_bytes"]
        n = shape.n_shared if shared else W.num_blobs(shape)
        self.host = torch.empty(max(n, 1), self.stride, dtype=torch.uint8, pin_memory=True)
        for b in range(n):
            w = (W.shared_expert_weights if shared else W.expert_weights)(shape, b, device=gen_device)
            B.moe_pack_expert_host(weights_to_host(w), shape.H, shape.F, self.wcode, self.host[b])
            del w
        self.n = n

    def row_ptr(self, blob: int) -> int:
        return self.host[blob].data_ptr()


@dataclass
class StepStats:
    hits: int = 0
    misses: int = 0
    fills: int = 0
    waves: int = 0
    distinct: int = 0


class SlotCacheLayer:
    """Slot pool, tables, routers and buffers of one workload on one GPU."""

    def __init__(self, shape: W.MoEShape, slots: int, residency: list, t_max: int,
                 store: ExpertStore | None = None, device="cuda"):
        self.shape, self.S, self.t_max, self.device = shape, slots, t_max, device
        sh = shape
        self.E, self.k, self.H, self.F, self.L = sh.E, sh.k, sh.H, sh.F, sh.layers
        self.store = store or ExpertStore(sh)
        self.stride, self.wcode = self.store.stride, self.store.wcode
        dev = torch.device(device)
        self.pool = torch.empty(slots * self.stride, dtype=torch.uint8, device=dev)
        self.lut = torch.full((self.L * self.E,), -1, dtype=torch.int32, device=dev)
        self.owner = torch.full((slots,), -1, dtype=torch.int32, device=dev)
        self.tags = torch.zeros(slots, dtype=torch.int64, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        # host mirror of the tables for the LRU plan
        self.lut_h = np.full(self.L * self.E, -1, np.int32)
        self.owner_h = np.full(slots, -1, np.int32)
        self.last_use_h = np.zeros(slots, np.int64)
        self.clock_h = np.zeros(1, np.int64)
        self.next_tag = 1
        self.fill_stream = torch.cuda.Stream(device=dev)
        self.routers = [W.router(sh, layer=l, device=dev) for l in range(self.L)]
        # buffers
        tk = t_max * self.k
        self.logits = torch.empty(t_max, self.E, dtype=torch.float32, device=dev)
        self.ids = torch.empty(t_max, self.k, dtype=torch.int32, device=dev)
        self.topw = torch.empty(t_max, self.k, dtype=torch.float32, device=dev)
        self.y_perm = torch.zeros(max(tk, 1), self.H, dtype=torch.float32, device=dev)
        ws = B.moe_ffn_workspace_bytes(t_max, self.H, self.F, self.E, self.k, self.wcode)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.masks = torch.zeros(64, self.E, dtype=torch.int32, device=dev)
        self.masks_h = torch.zeros(64, self.E, dtype=torch.int32, pin_memory=True)
        self.dist_h = torch.zeros(self.E + 1, dtype=torch.int32, pin_memory=True)
        self.dist_d = torch.zeros(self.E + 1, dtype=torch.int32, device=dev)
        self.perm = {n: torch.zeros(c, dtype=torch.int32, device=dev) for n, c in (
            ("counts", self.E), ("offsets", self.E + 1), ("perm", max(tk, 1)), ("inv", max(tk, 1)),
            ("distinct", self.E), ("n_distinct", 1))}
        # shared experts: resident pool of their own, identity table
        self.n_sh = sh.n_shared
        if self.n_sh:
            self.sh_store = ExpertStore(sh, shared=True)
            self.sh_pool = torch.empty(self.n_sh * self.stride, dtype=torch.uint8, device=dev)
            for s in range(self.n_sh):
                self.sh_pool[s * self.stride:(s + 1) * self.stride].copy_(self.sh_store.host[s])
            self.sh_lut = torch.arange(self.n_sh, dtype=torch.int32, device=dev)
            self.sh_y = torch.zeros(self.n_sh * t_max, self.H, dtype=torch.float32, device=dev)
            ws = B.moe_ffn_workspace_bytes(t_max, self.H, self.F, self.n_sh, self.n_sh, self.wcode)
            self.sh_ws = torch.empty(ws, dtype=torch.uint8, device=dev)
            self._sh_perm = {}
        for s, o in enumerate(residency):
            if o is not None:
                self._place(s, o[0], o[1])
        torch.cuda.synchronize()

    # -------------------------------------------------------------- filling
    def blob(self, layer: int, expert: int) -> int:
        return W.blob_of(self.shape, layer, expert)

    def _fill(self, slot: int, layer: int, expert: int, fill_stream, compute_stream):
        tag = self.next_tag
        self.next_tag += 1
        B.slot_fill(self.pool, self.stride, slot, self.store.row_ptr(self.blob(layer, expert)),
                    self.stride, self.lut, layer * self.E + expert, self.owner, self.tags, tag,
                    self.err, fill_stream=fill_stream, compute_stream=compute_stream)

    def _place(self, slot: int, layer: int, expert: int):
        """Initial residency: fill and mirror on the host table."""
        cs = torch.cuda.current_stream()
        self._fill(slot, layer, expert, cs, cs)
        idx = layer * self.E + expert
        old = self.owner_h[slot]
        if old >= 0:
            self.lut_h[old] = -1
        self.lut_h[idx] = slot
        self.owner_h[slot] = idx

    def shared_perm(self, T: int):
        if T not in self._sh_perm:
            n = self.n_sh
            perm = torch.tensor([t * n + s for s in range(n) for t in range(T)], dtype=torch.int32)
            offs = torch.tensor([s * T for s in range(n + 1)], dtype=torch.int32)
            self._sh_perm[T] = (perm.to(self.device), offs.to(self.device))
        return self._sh_perm[T]

    # ----------------------------------------------------------------- step
    def forward(self, x: torch.Tensor, layer: int = 0, out: torch.Tensor | None = None,
                stats: StepStats | None = None, ffn_events: list | None = None) -> torch.Tensor:
        """One layer step. ``ffn_events`` (optional list) receives a (start, end)
        pair of events recorded on the compute stream around every routed
        moe_expert_ffn call, with the number of expert groups it ran."""
        T = x.shape[0]
        assert T <= self.t_max
        E, k, H, F = self.E, self.k, self.H, self.F
        cs = torch.cuda.current_stream()
        wr, bias = self.routers[layer]
        B.moe_route(x, wr, bias, k, True, self.logits[:T], self.ids[:T], self.topw[:T])
        B.moe_permute(self.ids[:T], E, out=self.perm)
        # the distinct routed set goes to the host for the residency plan
        self.dist_d[:E].copy_(self.perm["distinct"])
        self.dist_d[E:].copy_(self.perm["n_distinct"])
        self.dist_h.copy_(self.dist_d, non_blocking=True)
        cs.synchronize()
        nd = int(self.dist_h[E])
        distinct = self.dist_h[:nd].numpy()
        plan = B.moe_plan_fills(self.lut_h, self.owner_h, self.last_use_h, self.clock_h, self.S,
                                self.L, E, layer, distinct)
        nw = plan["n_waves"]
        # masks: row 0 = hits, row 1 + w = filled groups of wave w
        m = self.masks_h
        m[:nw + 1].zero_()
        wave_of, is_hit = plan["wave_of"], plan["is_hit"]
        for e in distinct:
            if is_hit[e]:
                m[0, e] = 1
            else:
                m[1 + wave_of[e], e] = 1
        self.masks[:nw + 1].copy_(m[:nw + 1], non_blocking=True)
        lut_row = self.lut[layer * E:(layer + 1) * E]
        ev = torch.cuda.Event()
        ev.record(cs)
        self.fill_stream.wait_event(ev)
        def ffn(mask, groups):
            if ffn_events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(cs)
            B.moe_expert_ffn(x, self.perm["perm"], self.perm["offsets"], lut_row, mask, self.pool,
                             self.stride, self.wcode, T, H, F, E, k, self.y_perm, self.err, self.ws)
            if ffn_events is not None:
                e1.record(cs)
                ffn_events.append((e0, e1, groups))

        ffn(self.masks[0], int(is_hit.sum()))
        fe, fs, fw = plan["fill_expert"], plan["fill_slot"], plan["fill_wave"]
        for w in range(nw):
            if w > 0:  # the next wave overwrites slots the previous waves read
                ev = torch.cuda.Event()
                ev.record(cs)
                self.fill_stream.wait_event(ev)
            sel = np.flatnonzero(fw == w)
            for i in sel:
                self._fill(int(fs[i]), layer, int(fe[i]), self.fill_stream, cs)
            ffn(self.masks[1 + w], len(sel))
        shared_y = None
        if self.n_sh:
            sp, so = self.shared_perm(T)
            B.moe_expert_ffn(x, sp, so, self.sh_lut, None, self.sh_pool, self.stride, self.wcode, T, H,
                             F, self.n_sh, self.n_sh, self.sh_y, self.err, self.sh_ws)
            shared_y = self.sh_y[:self.n_sh * T].view(self.n_sh, T, H)
        out_dtype = torch.float32 if self.shape.xfmt == "f32" else torch.bfloat16
        out = B.moe_combine(self.y_perm, self.perm["inv"], self.topw[:T], T, k, H, shared_y, out,
                            out_dtype)
        if stats is not None:
            stats.distinct += nd
            stats.hits += int(is_hit.sum())
            stats.misses += len(fe)
            stats.fills += len(fe)
            stats.waves += nw
        return out
