"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark. It only draws random tensors of the shapes and distributions the
workloads need and rounds them to their storage dtype; it holds none of the
layer's arithmetic (no projection, gating, permutation, expert FFN, quantised
dot product or combine).

Conventions of every tensor produced here (nn.Linear orientation, row-major):
  tokens            x       [T, H]        fp32 or bf16
  router weight     w_r     [E, H]        row e is expert e's projection vector
  router bias       b       [E]           fp32 (Zipf skew; zeros when unskewed)
  expert weights    gate    [F, H], up [F, H], down [H, F]   (fp32 or bf16)
  int4 experts      *_q     uint8 [rows, K/2]: two signed 4-bit codes per byte
                            along K, even K index in the low nibble
                    *_s     bf16 [rows, K/128]: one scale per 128 K values
  split-precision   gate, up, down in fp32 (the masters the split-precision
  experts           quantiser reads; see the library's moe_quantize_resplit_host)

Large tensors are drawn with torch's seeded generator on the device given, so
the full-size workloads can be produced on the GPU in seconds; the values then
depend only on (seed, device type).
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class MoEShape:
    """Shape and data recipe of one routed-expert layer (or a stack of them)."""

    name: str
    E: int                      # routed experts per layer
    k: int                      # experts selected per token
    H: int                      # hidden size
    F: int                      # expert FFN (intermediate) size
    n_shared: int = 0           # always-on shared experts (weight 1, resident)
    wfmt: str = "bf16"          # expert weight storage: "f32" | "bf16" | "int4g128" |
                                # "int4g128_resplit" (fp32 masters, split-precision slots)
    xfmt: str = "bf16"          # tokens and router weight: "f32" | "bf16"
    zipf_s: float | None = None  # Zipf exponent of the per-expert logit bias
    layers: int = 1
    blobs: int | None = None    # distinct weight sets backing the layer-experts
    ar_rho: float | None = None  # step-to-step correlation of a layer's input
    w_std: float = 0.02         # standard deviation of synthetic weights

    @property
    def is_int4(self) -> bool:
        return self.wfmt == "int4g128"


# The five workloads, named by what they are and their sizes.
WORKLOADS: dict[str, dict] = {
    "tiny_e8k2_h256_f512_fp32": dict(
        shape=MoEShape("tiny_e8k2_h256_f512_fp32", E=8, k=2, H=256, F=512,
                       wfmt="f32", xfmt="f32", zipf_s=1.1),
        tokens=[16], slots=[8], residency="identity"),
    "mixtral_e8k2_h4096_f14336_bf16": dict(
        shape=MoEShape("mixtral_e8k2_h4096_f14336_bf16", E=8, k=2, H=4096, F=14336),
        tokens=[1, 8, 512], slots=[4], residency="random"),
    "qwen3moe_l48_e128k8_h2048_f768_bf16": dict(
        shape=MoEShape("qwen3moe_l48_e128k8_h2048_f768_bf16", E=128, k=8, H=2048, F=768,
                       zipf_s=1.2, layers=48, blobs=128, ar_rho=0.7),
        tokens=[1, 16], slots=[2765], residency="zipf_rank", steps=64),
    "dsv2lite_e64k6s2_h2048_f1408_bf16": dict(
        shape=MoEShape("dsv2lite_e64k6s2_h2048_f1408_bf16", E=64, k=6, H=2048, F=1408,
                       n_shared=2, zipf_s=1.0),
        tokens=[1, 32, 256, 1024], slots=[16, 32, 48], residency="zipf_rank"),
    "dsv3_e256k8s1_h7168_f2048_int4": dict(
        shape=MoEShape("dsv3_e256k8s1_h7168_f2048_int4", E=256, k=8, H=7168, F=2048,
                       n_shared=1, wfmt="int4g128", zipf_s=1.1),
        tokens=[1, 32, 4096], slots=[84], residency="zipf_rank"),
}


def shape_of(name: str) -> MoEShape:
    return WORKLOADS[name]["shape"]


# ---------------------------------------------------------------- seeding ---
_KIND = {"x": 1, "router": 2, "expert": 3, "zipf_perm": 4, "residency": 5,
         "ar": 6, "shared": 7, "bias_noise": 8}


def seed_for(shape: MoEShape, kind: str, *idx: int) -> int:
    """63-bit seed derived from seed 0, the workload name and the tensor's role."""
    ss = np.random.SeedSequence(
        entropy=0, spawn_key=(zlib.crc32(shape.name.encode()), _KIND[kind], *map(int, idx)))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(shape: MoEShape, kind: str, *idx: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_for(shape, kind, *idx))
    return g


def _tdtype(fmt: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "int4g128_resplit": torch.float32}[fmt]


# ---------------------------------------------------------------- tensors ---
def tokens(shape: MoEShape, T: int, *, layer: int = 0, step: int = 0, device="cpu") -> torch.Tensor:
    """x ~ N(0, 1), [T, H], rounded (RNE) to the activation dtype."""
    g = _gen(shape, "x", layer, step, T, device=device)
    x = torch.randn(T, shape.H, generator=g, device=device, dtype=torch.float32)
    return x.to(_tdtype(shape.xfmt))


def token_sequence(shape: MoEShape, T: int, steps: int, *, layer: int = 0, device="cpu") -> torch.Tensor:
    """[steps, T, H] layer inputs with AR(1) correlation ``ar_rho`` between steps.

    x_0 = eps_0, x_s = rho * x_{s-1} + sqrt(1 - rho^2) * eps_s, eps ~ N(0, 1),
    drawn in fp32 and rounded to the activation dtype at the end.
    """
    rho = shape.ar_rho if shape.ar_rho is not None else 0.0
    g = _gen(shape, "ar", layer, T, steps, device=device)
    eps = torch.randn(steps, T, shape.H, generator=g, device=device, dtype=torch.float32)
    out = torch.empty_like(eps)
    out[0] = eps[0]
    c = math.sqrt(1.0 - rho * rho)
    for s in range(1, steps):
        out[s] = rho * out[s - 1] + c * eps[s]
    return out.to(_tdtype(shape.xfmt))


def zipf_permutation(shape: MoEShape, layer: int = 0) -> torch.Tensor:
    """pi: seeded permutation of the experts; expert e has Zipf rank 1 + pi[e]."""
    g = _gen(shape, "zipf_perm", layer)
    return torch.randperm(shape.E, generator=g)


def router(shape: MoEShape, *, layer: int = 0, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """Router weight [E, H] ~ N(0, w_std) in the activation dtype, and bias [E] fp32.

    The bias carries the routing skew: b_e = -s * ln(1 + pi[e]), so that the
    prior selection odds of expert e fall off as rank^-s (Zipf). No skew: zeros.
    """
    g = _gen(shape, "router", layer, device=device)
    w = (torch.randn(shape.E, shape.H, generator=g, device=device, dtype=torch.float32)
         * shape.w_std).to(_tdtype(shape.xfmt))
    if shape.zipf_s is None:
        b = torch.zeros(shape.E, dtype=torch.float32)
    else:
        rank = zipf_permutation(shape, layer).to(torch.float64) + 1.0
        b = (-shape.zipf_s * torch.log(rank)).to(torch.float32)
    return w, b.to(device)


def _dense_expert(shape: MoEShape, g: torch.Generator, device) -> dict[str, torch.Tensor]:
    dt = _tdtype(shape.wfmt)
    H, F = shape.H, shape.F
    out = {}
    for name, (r, c) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        out[name] = (torch.randn(r, c, generator=g, device=device, dtype=torch.float32)
                     * shape.w_std).to(dt)
    return out


# Uniform 4-bit codes on [-8, 7] have standard deviation sqrt((16^2 - 1) / 12).
_INT4_CODE_STD = math.sqrt((16 * 16 - 1) / 12.0)


def _int4_expert(shape: MoEShape, g: torch.Generator, device) -> dict[str, torch.Tensor]:
    """Synthetic int4 group-128 expert: random codes and bf16 scales.

    Codes are uniform over the 16 signed values; each group scale is
    w_std / code_std times a factor uniform in [0.75, 1.25), so the dequantised
    weights have roughly the w_std spread and every group has its own scale.
    """
    H, F = shape.H, shape.F
    base = shape.w_std / _INT4_CODE_STD
    out = {}
    for name, (r, c) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        out[name + "_q"] = torch.randint(0, 256, (r, c // 2), generator=g, device=device,
                                         dtype=torch.uint8)
        u = torch.rand(r, c // 128, generator=g, device=device, dtype=torch.float32)
        out[name + "_s"] = (base * (0.75 + 0.5 * u)).to(torch.bfloat16)
    return out


def expert_weights(shape: MoEShape, blob: int, *, device="cpu") -> dict[str, torch.Tensor]:
    """Weights of routed weight set ``blob`` (see ``blob_of``)."""
    g = _gen(shape, "expert", blob, device=device)
    return _int4_expert(shape, g, device) if shape.is_int4 else _dense_expert(shape, g, device)


def shared_expert_weights(shape: MoEShape, j: int, *, device="cpu") -> dict[str, torch.Tensor]:
    g = _gen(shape, "shared", j, device=device)
    return _int4_expert(shape, g, device) if shape.is_int4 else _dense_expert(shape, g, device)


def blob_of(shape: MoEShape, layer: int, expert: int) -> int:
    """Weight set that backs (layer, expert).

    Without aliasing every layer-expert has its own set. With ``blobs`` sets
    (a stack whose full host store would not fit), layer l maps expert e to
    set (e + 37 l) mod blobs, a bijection inside each layer when blobs == E.
    """
    if shape.blobs is None:
        return layer * shape.E + expert
    return (expert + 37 * layer) % shape.blobs


def num_blobs(shape: MoEShape) -> int:
    return shape.layers * shape.E if shape.blobs is None else shape.blobs


def initial_residency(shape: MoEShape, slots: int, mode: str) -> list[tuple[int, int] | None]:
    """Initial owner of each slot: (layer, expert) or None (empty slot).

    identity:  slot s holds expert s of layer 0.
    random:    ``slots`` experts of layer 0 drawn without replacement, in the
               drawn order, so the expert->slot map is a random relabelling.
    zipf_rank: each layer gets slots // layers experts (the first
               slots % layers layers one more), taken by ascending Zipf rank;
               slot ids are assigned layer-major. Stands in for an offline
               activation-frequency profile.
    """
    if mode == "identity":
        return [(0, s) if s < shape.E else None for s in range(slots)]
    if mode == "random":
        rng = np.random.Generator(np.random.PCG64(seed_for(shape, "residency", slots)))
        chosen = rng.choice(shape.E, size=min(slots, shape.E), replace=False)
        own = [(0, int(e)) for e in chosen]
        return own + [None] * (slots - len(own))
    if mode == "zipf_rank":
        per, extra = divmod(slots, shape.layers)
        own: list[tuple[int, int] | None] = []
        for layer in range(shape.layers):
            n = min(shape.E, per + (1 if layer < extra else 0))
            by_rank = torch.argsort(zipf_permutation(shape, layer)).tolist()
            own += [(layer, int(e)) for e in by_rank[:n]]
        return own + [None] * (slots - len(own))
    raise ValueError(mode)


def reduced(shape: MoEShape, **kw) -> MoEShape:
    """Same recipe at other sizes (parity cases the oracle finishes in seconds)."""
    d = {f: getattr(shape, f) for f in shape.__dataclass_fields__}
    d.update(kw)
    if "name" not in kw:
        d["name"] = shape.name + "_reduced_" + "_".join(f"{a}{b}" for a, b in sorted(kw.items()))
    return MoEShape(**d)
