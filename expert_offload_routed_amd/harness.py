"""Device state of one routed-expert workload on one GPU, driving the native runtime.

PyTorch provides device memory, pinned host memory and streams. A layer step
is one call of moe_layer_forward (include/moe_runtime.h). Inside libmoe_offload
it runs the route and permutation, the eviction plan (LRU, Minus Recent Score
or routing history; on the host, or on the GPU under device orchestration),
the expert FFN over resident slots overlapped with tagged fills of the misses,
the shared experts, and the combine as its own launch.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B
from . import workloads as W

WFMT_CODE = {"f32": B.MOE_F32, "bf16": B.MOE_BF16, "int4g128": B.MOE_INT4G128,
             "int4g128_resplit": B.MOE_INT4G128_RESPLIT}


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
            if self.wcode == B.MOE_INT4G128_RESPLIT:  # quantised from the fp32 masters
                B.moe_quantize_resplit_host(w["gate"], w["up"], w["down"], shape.H, shape.F,
                                            self.host[b])
            else:
                B.moe_pack_expert_host(weights_to_host(w), shape.H, shape.F, self.wcode,
                                       self.host[b])
            del w
        self.n = n

    def row_ptr(self, blob: int) -> int:
        return self.host[blob].data_ptr()


@dataclass
class StepStats:
    steps: int = 0


class SlotCacheLayer:
    """Slot pool, tables, routers and the native layer runtime of one workload on one GPU.

    Memory comes from torch (device pool, tables, workspace; pinned host
    store); each step is one moe_layer_forward call into libmoe_offload.
    """

    def __init__(self, shape: W.MoEShape, slots: int, residency: list, t_max: int,
                 store: ExpertStore | None = None, device="cuda", compute_stream=None,
                 staging: bool = False):
        self.shape, self.S, self.t_max, self.device = shape, slots, t_max, device
        sh = shape
        self.E, self.k, self.H, self.F, self.L = sh.E, sh.k, sh.H, sh.F, sh.layers
        self.store = store or ExpertStore(sh)
        self.stride, self.wcode = self.store.stride, self.store.wcode
        dev = torch.device(device)
        self.n_sh = sh.n_shared
        # the S routed slots, then the n_shared slots of the always-resident shared experts,
        # then (staging) two buffers of E slots for prefill full-layer staging
        self.pool_slots = slots + self.n_sh + (2 * self.E if staging else 0)
        self.pool = torch.empty(self.pool_slots * self.stride, dtype=torch.uint8, device=dev)
        self.lut = torch.full((self.L * self.E,), -1, dtype=torch.int32, device=dev)
        self.owner = torch.full((slots,), -1, dtype=torch.int32, device=dev)
        self.tags = torch.zeros(slots, dtype=torch.int64, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.routers = [W.router(sh, layer=l, device=dev) for l in range(self.L)]
        self.sh_pool = None
        if self.n_sh:
            self.sh_store = ExpertStore(sh, shared=True)
            self.sh_pool = self.pool[slots * self.stride:(slots + self.n_sh) * self.stride]
            for s in range(self.n_sh):
                self.sh_pool[s * self.stride:(s + 1) * self.stride].copy_(self.sh_store.host[s])
        blob_of = np.array([W.blob_of(sh, l, e) for l in range(self.L) for e in range(self.E)], np.int32)
        xcode = B.MOE_F32 if sh.xfmt == "f32" else B.MOE_BF16
        self.ctx = B.LayerContext(
            t_max=t_max, H=self.H, F=self.F, E=self.E, k=self.k, L=self.L, S=slots, x_dtype=xcode,
            w_dtype=self.wcode, n_shared=self.n_sh, pool=self.pool, slot_stride=self.stride,
            lut=self.lut, owner=self.owner, tags=self.tags, host_store=self.store.host,
            blob_of=blob_of, shared_pool=self.sh_pool, err=self.err, compute_stream=compute_stream)
        for s, o in enumerate(residency):
            if o is not None:
                self.ctx.place(s, o[0], o[1])
        self.out_dtype = torch.float32 if sh.xfmt == "f32" else torch.bfloat16
        self._st = np.zeros(4, np.int32)
        torch.cuda.synchronize()

    def forward(self, x: torch.Tensor, layer: int = 0, out: torch.Tensor | None = None,
                stats: StepStats | None = None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=self.out_dtype, device=x.device)
        wr, bias = self.routers[layer]
        self.ctx.forward(layer, x, wr, bias, out, self._st)
        if stats is not None:
            stats.steps += 1
        return out

    def forward_steps(self, steps, out: torch.Tensor) -> None:
        """Run [(layer, x), ...] in order with one native call; every step writes `out`."""
        code = B.dtype_code(out)
        self.ctx.forward_steps([(l, x, self.routers[l][0], self.routers[l][1], out) for l, x in steps], code)

    def counters(self) -> dict:
        return self.ctx.counters()

    def outputs(self, T: int) -> dict:
        return self.ctx.outputs(T)

    def tables(self):
        return self.ctx.tables()
