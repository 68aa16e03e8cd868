"""Oracle functions, one per step of the routed-expert layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): not imported by the
product path.

Sources, cited by page title and section:
  [RapidMoE]  "RapidMoE: Exploiting Cross-Asymmetry via Adaptive Residual
              Offloading for Large-Scale MoE Inference", Sec. 2.1 (gating,
              top-k, weighted sum), Algorithm 1 (weighted sum over the routed
              experts), Sec. 4.4-4.5 and Eq. (7) (SwiGLU expert).
              Sec. 4.2 and Eqs. (3)-(5) (critical set by a multi-modulated
              threshold on the router scores), Algorithm 1 (critical experts
              on high-precision weights, the rest on low-precision ones),
              Sec. 4.4 and Algorithm 3 (residual split of gate/up, two
              separate quantisations of down).
  [CAP]       "Communication-Aware Placement and Pruning for Efficient
              Mixture-of-Experts Inference", Sec. II-A, Eq. (1) (normalised
              routing weights).
  [SeqMoE]    SeqMoE summary page (graph-compatible MoE offload), Mechanism:
              one slot pool at a fixed base, expert_id -> slot_id table,
              pinned host pool, per-slot tags.
  [HybriMoE]  HybriMoE summary page (hybrid CPU-GPU scheduling), Mechanism:
              misses = routed set minus cached set; only routed experts cached;
              LRU as the baseline replacement.
  [MoE-CORE]  MoE-CORE summary page (coordinated expert offload), Mechanism:
              routed experts in a fixed-budget device cache; eviction by a
              routing-history score.

Readings of points the pages leave open (each also listed in the design notes):
  * selection is on the logits (same set as on softmax probabilities), ties go
    to the lower expert id, selected ids are ordered by descending logit;
  * the bias is part of the logit (added before selection and softmax);
  * gate weights are the softmax probabilities of the selected experts divided
    by their sum (renormalised); with renorm off they are the plain softmax
    probabilities;
  * SiLU is applied to the gate projection only: h = SiLU(x W_gate) * (x W_up)
    (Eq. (7) in [RapidMoE]; its Sec. 4.4 text is garbled on this point);
  * int4 weights are symmetric with one bf16 scale per 128 input values;
    int8 activations use one fp32 scale per row, absmax / 127;
  * a term whose gate weight is exactly zero is skipped in the weighted sum;
  * the routing score of an expert at a step is its softmax probability
    averaged over the step's tokens; eviction scores are kept per layer and
    compared across layers as they stand.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

try:  # torch tensors are accepted as inputs; the oracle computes in numpy.
    import torch
except ImportError:  # pragma: no cover
    torch = None

__all__ = [
    "as_f64", "as_f32", "router_logits", "select_topk", "topk_margin", "gate_weights",
    "permute", "silu", "swiglu_expert", "decode_int4", "dequant_int4g128",
    "quantize_rows_int8", "swiglu_expert_w4a8", "expert_forward", "combine",
    "SlotPool", "LruSlotPlanner", "Wave", "route", "moe_layer",
    "step_scores", "MinusRecentScore", "RoutingHistoryScore", "ScoredSlotPlanner",
    "round_bf16", "quantize_sym_g128", "resplit_expert", "critical_threshold",
    "critical_experts", "swiglu_expert_split", "prefetch_window", "prefetch_count",
    "prefetch_candidates",
]


# ------------------------------------------------------------ conversions ---
def as_f64(a) -> np.ndarray:
    """Exact float64 copy of a float32/bf16 array (torch bf16 -> fp32 is exact)."""
    if torch is not None and isinstance(a, torch.Tensor):
        a = a.detach().to("cpu")
        if a.dtype == torch.bfloat16:
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def as_f32(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        a = a.detach().to("cpu")
        if a.dtype == torch.bfloat16:
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float32)


def _np(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu").numpy()
    return np.asarray(a)


# ---------------------------------------------------------------- routing ---
def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Router logits l[t, e] = sum_h x[t, h] * w_r[e, h] + b[e], float64.

    [RapidMoE] Sec. 2.1: the gating function is a linear projection of the
    token followed by softmax; the bias carries the synthetic routing skew.
    """
    x64, w64 = as_f64(x), as_f64(w_router)
    logits = x64 @ w64.T
    if bias is not None:
        logits = logits + as_f64(bias)[None, :]
    return logits


def select_topk(scores, k: int) -> np.ndarray:
    """ids[t, :] = the first k experts in the order (score descending, id ascending).

    [RapidMoE] Sec. 2.1: the k experts with the highest logits are activated.
    The comparison is exact on whatever precision ``scores`` holds; callers
    pass float32 scores so that the decision is taken in the kernels'
    precision.
    """
    s = np.asarray(scores)
    T, E = s.shape
    ids = np.empty((T, k), dtype=np.int32)
    expert = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> descending score, then ascending id.
        order = np.lexsort((expert, -s[t]))
        ids[t] = order[:k]
    return ids


def topk_margin(scores, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest score of each token (inf if k == E)."""
    s = np.sort(np.asarray(scores, dtype=np.float64), axis=1)[:, ::-1]
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def gate_weights(logits, ids, renorm: bool = True) -> np.ndarray:
    """Routing weights of the selected experts, float64.

    p = softmax over all experts (max-subtracted); w[t, j] = p[t, ids[t, j]],
    divided by the sum over the k selected when ``renorm`` ([CAP] Eq. (1):
    normalised routing weight of each selected expert).
    """
    l64 = as_f64(logits)
    m = l64.max(axis=1, keepdims=True)
    p = np.exp(l64 - m)
    p = p / p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(x, w_router, bias, k: int, renorm: bool = True) -> dict:
    """Logits (float64), their float32 rounding, selection on the float32 values, weights."""
    logits = router_logits(x, w_router, bias)
    logits32 = logits.astype(np.float32)
    ids = select_topk(logits32, k)
    return dict(logits=logits, logits32=logits32, ids=ids,
                weights=gate_weights(logits, ids, renorm), margin=topk_margin(logits32, k))


# ------------------------------------------------------------ permutation ---
def permute(ids, E: int) -> dict:
    """Counting sort of the T*k assignments by expert, stable in token order.

    Flat assignment index f = t*k + j. For each expert in ascending id, the
    flat indices routed to it in ascending order; counts, exclusive offsets,
    perm (sorted position -> f), inv (f -> sorted position) and the distinct
    routed experts (count > 0, ascending).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    perm: list[int] = []
    for e in range(E):
        rows = np.flatnonzero(flat == e)
        counts[e] = rows.size
        offsets[e + 1] = offsets[e] + rows.size
        perm.extend(int(r) for r in rows)
    perm_a = np.asarray(perm, dtype=np.int32)
    inv = np.empty(flat.size, dtype=np.int32)
    for pos, f in enumerate(perm_a):
        inv[f] = pos
    distinct = np.asarray([e for e in range(E) if counts[e] > 0], dtype=np.int32)
    return dict(counts=counts, offsets=offsets, perm=perm_a, inv=inv, distinct=distinct)


# -------------------------------------------------------------- expert FFN ---
def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_expert(x_rows, gate, up, down) -> np.ndarray:
    """One expert on a block of rows: y = (SiLU(x W_gate) * (x W_up)) W_down.

    [RapidMoE] Eq. (7): SiLU acts on the gate projection, the product with the
    up projection feeds the down projection. Weights are in nn.Linear
    orientation: gate, up [F, H]; down [H, F].
    """
    x64 = as_f64(x_rows)
    g = x64 @ as_f64(gate).T
    u = x64 @ as_f64(up).T
    with np.errstate(over="ignore"):
        h = silu(g) * u
    return h @ as_f64(down).T


# the two signed 4-bit codes of each byte value: low nibble first; a nibble v
# in [0, 16) stands for the two's-complement value (v ^ 8) - 8
_NIBBLE_PAIRS = np.array([[((b & 15) ^ 8) - 8, ((b >> 4) ^ 8) - 8] for b in range(256)],
                         dtype=np.int8)


def decode_int4(codes) -> np.ndarray:
    """Packed signed 4-bit codes [rows, K/2] (even K in the low nibble) -> int8 [rows, K]."""
    b = _np(codes).astype(np.uint8)
    return _NIBBLE_PAIRS[b].reshape(b.shape[0], b.shape[1] * 2)


def dequant_int4g128(codes, scales) -> np.ndarray:
    """W_hat[n, c] = q[n, c] * s[n, c // 128] (exact in float64)."""
    q = decode_int4(codes)
    s = as_f64(scales)
    rows, K = q.shape
    return (q.reshape(rows, K // 128, 128).astype(np.float64) * s[:, :, None]).reshape(rows, K)


def quantize_rows_int8(a) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row int8: s = max|a_row| / 127, q = clip(rint(a / s), -127, 127).

    Taken in float32 (the kernels' precision), since the float result decides
    an integer code; a zero row gets s = 1 and q = 0.
    """
    a32 = as_f32(a)
    amax = np.max(np.abs(a32), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = np.clip(np.rint(a32 / s[:, None]), -127, 127).astype(np.int8)
    return q, s


def swiglu_expert_w4a8(x_rows, w: dict) -> np.ndarray:
    """SwiGLU expert with int4 group-128 weights and int8 per-row activations.

    x rows and the SwiGLU intermediate are each quantised per row to int8
    (float32 decision), dequantised exactly, and multiplied in float64 by the
    exactly dequantised int4 weights.
    """
    qx, sx = quantize_rows_int8(x_rows)
    xh = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    g = xh @ dequant_int4g128(w["gate_q"], w["gate_s"]).T
    u = xh @ dequant_int4g128(w["up_q"], w["up_s"]).T
    with np.errstate(over="ignore"):
        h = silu(g) * u
    qh, sh = quantize_rows_int8(h.astype(np.float32))
    hh = qh.astype(np.float64) * sh.astype(np.float64)[:, None]
    return hh @ dequant_int4g128(w["down_q"], w["down_s"]).T


def expert_forward(x_rows, w: dict, critical: bool = True) -> np.ndarray:
    """One expert on a block of rows, in the form its weights are stored: split
    precision (at W^H when ``critical``, else W^L), int4 group-128 with int8
    rows, or dense fp32/bf16 values."""
    if "down_lq" in w:
        return swiglu_expert_split(x_rows, w, critical)
    if "gate_q" in w:
        return swiglu_expert_w4a8(x_rows, w)
    return swiglu_expert(x_rows, w["gate"], w["up"], w["down"])


# ---------------------------------------------------------------- combine ---
def combine(y_assign, weights, shared=None) -> np.ndarray:
    """out[t] = sum_j [w[t,j] != 0] w[t,j] * y[t,j] + sum_s y_shared[s, t].

    [RapidMoE] Sec. 2.1 and Algorithm 1: weighted sum of the routed experts'
    outputs; [CAP] Eq. (1). y_assign is [T, k, H]: the output of the expert
    routed at (t, j) for token t. Shared experts enter with weight 1.
    """
    y = as_f64(y_assign)
    w = as_f64(weights)
    T, k, H = y.shape
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        nz = w[:, j] != 0.0
        out[nz] += w[nz, j, None] * y[nz, j]
    if shared is not None:
        for ys in shared:
            out += as_f64(ys)
    return out


# -------------------------------------------------------------- slot pool ---
class SlotPool:
    """The fixed-base pool of expert slots and the expert_id -> slot_id table.

    [SeqMoE] Mechanism: one pool of slots shared by every MoE layer; a lookup
    table rewrites expert ids to slot ids, so the expert computation reads an
    expert's weights through its slot. Here a slot holds a reference to the
    weights last copied into it, and ``owner`` the (layer, expert) whose table
    entry points at it.
    """

    def __init__(self, num_slots: int, layers: int, E: int):
        self.content: list[dict | None] = [None] * num_slots
        self.owner: list[tuple[int, int] | None] = [None] * num_slots
        self.lut = np.full((layers, E), -1, dtype=np.int32)

    def commit(self, slot: int, layer: int, expert: int, weights: dict) -> None:
        """Copy an expert into a slot and point its table entry there; the
        slot's previous owner loses its entry (it is no longer resident)."""
        old = self.owner[slot]
        if old is not None:
            self.lut[old] = -1
        self.content[slot] = weights
        self.owner[slot] = (layer, expert)
        self.lut[layer, expert] = slot

    def weights_of(self, layer: int, expert: int) -> dict:
        slot = int(self.lut[layer, expert])
        if slot < 0:
            raise KeyError(f"expert {expert} of layer {layer} is not resident")
        return self.content[slot]


@dataclass
class Wave:
    compute: list[int]                                           # experts computed
    fills: list[tuple[int, int]] = field(default_factory=list)   # (expert, slot)


class LruSlotPlanner:
    """Residency plan for one layer call: hits, misses, victims, fill waves.

    The pages give the vocabulary ([HybriMoE] Mechanism: misses are the routed
    set minus the cached set, only routed experts are cached, LRU is the
    baseline replacement; [SeqMoE] Mechanism: one shared pool and a per-layer
    table) but no hot-path victim rule, so this is plain least-recently-used:

      U = distinct routed experts (ascending), H = resident ones, M = the rest.
      Victims: empty slots by ascending id, then slots not holding a member of
      H, by (last use, slot id) ascending.
      If |M| <= |victims|: one wave, M[i] goes to victim i.
      Otherwise: wave 1 computes H and the first (S - |H|) misses (into the
      victims); every later wave takes up to S further misses into slots
      0, 1, ... in order (the earlier waves' experts are already consumed).
      A clock advances once per call; every slot used in the call gets it as
      its last use. The table keeps the state after the last wave.
    """

    _victim_key = None  # ordering of the reusable slots; None = (last use, slot id)

    def __init__(self, num_slots: int, layers: int, E: int,
                 residency: list[tuple[int, int] | None] | None = None):
        if num_slots < 1:
            raise ValueError("need at least one slot")
        self.S, self.L, self.E = num_slots, layers, E
        self.lut = np.full((layers, E), -1, dtype=np.int32)
        self.owner: list[tuple[int, int] | None] = [None] * num_slots
        self.last_use = [0] * num_slots
        self.clock = 0
        for s, o in enumerate(residency or []):
            if o is not None:
                self.lut[o] = s
                self.owner[s] = o

    def _assign(self, layer: int, expert: int, slot: int) -> None:
        old = self.owner[slot]
        if old is not None:
            self.lut[old] = -1
        self.lut[layer, expert] = slot
        self.owner[slot] = (layer, expert)

    def plan(self, layer: int, distinct) -> list[Wave]:
        self.clock += 1
        U = sorted(int(e) for e in distinct)
        hits = [e for e in U if self.lut[layer, e] >= 0]
        misses = [e for e in U if self.lut[layer, e] < 0]
        kept = {int(self.lut[layer, e]) for e in hits}
        empty = [s for s in range(self.S) if self.owner[s] is None]
        key = self._victim_key or (lambda s: (self.last_use[s], s))
        reusable = sorted((s for s in range(self.S) if self.owner[s] is not None and s not in kept),
                          key=key)
        victims = empty + reusable
        used = set(kept)
        waves: list[Wave] = []
        if len(misses) <= len(victims):
            fills = list(zip(misses, victims))
            waves.append(Wave(compute=list(U), fills=fills))
        else:
            first = misses[:len(victims)]
            waves.append(Wave(compute=hits + first, fills=list(zip(first, victims))))
            rest = misses[len(first):]
            for i in range(0, len(rest), self.S):
                chunk = rest[i:i + self.S]
                waves.append(Wave(compute=list(chunk), fills=list(zip(chunk, range(len(chunk))))))
        for wave in waves:
            for e, s in wave.fills:
                self._assign(layer, e, s)
                used.add(s)
        for s in used:
            self.last_use[s] = self.clock
        return waves

    def prefetch(self, layer: int, pred_ids, pred_scores, window_us: float, bw_gbs: float,
                 expert_bytes: int) -> list[tuple[int, int]]:
        """Prefetch for the next layer's step, after the current step's plan ([MoE-CORE]
        Mechanism): the prefetch_candidates of `layer`, as many as prefetch_count allows,
        go to free slots in the victim order: empty slots first, then slots the current
        step did not use (last use before the clock) and that hold no predicted expert of
        `layer`. A prefetched slot gets the current clock as its last use (it waits for
        its step). Returns [(expert, slot)] in order."""
        cand = prefetch_candidates(pred_ids, pred_scores, self.lut[layer])
        pred = {int(e) for e in np.asarray(pred_ids).ravel()}
        empty = [s for s in range(self.S) if self.owner[s] is None]
        key = self._victim_key or (lambda s: (self.last_use[s], s))
        reusable = sorted((s for s in range(self.S)
                           if self.owner[s] is not None and self.last_use[s] < self.clock
                           and not (self.owner[s][0] == layer and self.owner[s][1] in pred)),
                          key=key)
        free = empty + reusable
        n = min(prefetch_count(window_us, bw_gbs, expert_bytes, len(free)), len(cand))
        out = []
        for e, s in zip(cand[:n], free[:n]):
            self._assign(layer, e, s)
            self.last_use[s] = self.clock
            out.append((e, s))
        return out


# ------------------------------------------------------- miss prefetch ---
def prefetch_window(t_remain_us: float, t_attn_us: float, t_launch_us: float) -> float:
    """[MoE-CORE] Mechanism: the time a prefetch copy can hide, the remaining compute of
    layer l plus the attention of layer l+1, minus the launch overhead (microseconds)."""
    return t_remain_us + t_attn_us - t_launch_us


def prefetch_count(window_us: float, bw_gbs: float, expert_bytes: int, free_slots: int) -> int:
    """[MoE-CORE] Mechanism: as many experts as the window can hide at the host-to-device
    bandwidth, floor(window * BW / expert bytes), further capped by the free slots; none
    when the window is not positive. float64 in this order (microseconds, GB/s, bytes)."""
    if not window_us > 0.0:
        return 0
    n = int(np.floor(window_us * bw_gbs * 1000.0 / float(expert_bytes)))
    return max(0, min(n, free_slots))


def prefetch_candidates(pred_ids, pred_scores, lut_row) -> list[int]:
    """[MoE-CORE] Mechanism: the next layer's router evaluated on the current hidden state
    predicts its routed set; the candidates are the predicted experts not resident, the
    top predicted first. Readings: the predicted set is the union of the tokens' top-k;
    "top" orders by the predicted routing score (the softmax probability averaged over the
    step's tokens, float32 as given), ties to the lower id."""
    sc = as_f32(pred_scores)
    pred = sorted({int(e) for e in np.asarray(pred_ids).ravel()})
    cand = [e for e in pred if lut_row[e] < 0]
    return sorted(cand, key=lambda e: (-float(sc[e]), e))


# --------------------------------------------------------- eviction scores ---
def step_scores(logits) -> np.ndarray:
    """Routing score of every expert at one step: its softmax probability over
    the step's tokens, averaged over the tokens ([RapidMoE] Sec. 2.1 softmax;
    the averaging over a batch is the reading for T > 1). fp64."""
    lg = as_f64(logits).reshape(-1, np.shape(logits)[-1])
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


class MinusRecentScore:
    """[HybriMoE] Mechanism, Minus Recent Score: the routing scores of an
    expert over the recent steps of its layer are added up and the most recent
    one is subtracted, so a single high score on the latest step does not
    protect the expert. The lowest score is evicted first.

    Readings: "recent steps" are the last `window` steps of the layer,
    including the current one; the sum runs from the oldest to the newest step
    in float64 and the newest score is then subtracted.
    """

    def __init__(self, layers: int, E: int, window: int):
        if window < 1:
            raise ValueError("window must be at least 1")
        self.W = window
        self.hist = [[] for _ in range(layers)]  # per layer: score vectors, oldest first

    def observe(self, layer: int, scores, distinct) -> None:
        h = self.hist[layer]
        h.append([float(v) for v in np.asarray(scores, dtype=np.float32)])
        if len(h) > self.W:
            h.pop(0)

    def keep(self, layer: int, expert: int) -> float:
        h = self.hist[layer]
        if not h:
            return 0.0
        total = 0.0
        for row in h:
            total += row[expert]
        return total - h[-1][expert]


class RoutingHistoryScore:
    """[MoE-CORE] Mechanism, routing-history eviction score: four features of
    an expert -- how often it was selected in a recent window, an exponential
    moving average of its selections, its current routing score, and its age
    since it was last selected -- each normalised across the experts of the
    layer, combined with nonnegative weights. The lowest score is evicted first.

    Readings: the window is the last `window` steps of the layer (the current
    one included); the moving average is ema <- lam * ema + (1 - lam) * [selected]
    over every step of the layer, starting at 0; the current score is the
    routing score of the latest step; a feature is normalised by dividing by its
    maximum over the layer (0 when that maximum is 0); age enters as freshness
    1 - age / max_age (age = steps of the layer since the last selection, the
    step count when never selected; freshness 1 when max_age is 0), so every
    weight rewards keeping. keep = w_cnt*cnt + w_ema*ema + w_score*score +
    w_fresh*fresh, summed in that order in float64.
    """

    def __init__(self, layers: int, E: int, window: int,
                 weights=(1.0, 1.0, 1.0, 1.0), lam: float = 0.9):
        if window < 1 or any(w < 0 for w in weights) or not 0.0 <= lam <= 1.0:
            raise ValueError("bad routing-history parameters")
        self.W, self.E = window, E
        self.w = [float(v) for v in weights]
        self.lam = float(lam)
        self.steps = [0] * layers
        self.sel = [[] for _ in range(layers)]        # per layer: selection sets, oldest first
        self.ema = [[0.0] * E for _ in range(layers)]
        self.score = [[0.0] * E for _ in range(layers)]
        self.last = [[0] * E for _ in range(layers)]  # step of the last selection, 0 = never

    def observe(self, layer: int, scores, distinct) -> None:
        self.steps[layer] += 1
        n = self.steps[layer]
        chosen = {int(e) for e in distinct}
        self.sel[layer].append(chosen)
        if len(self.sel[layer]) > self.W:
            self.sel[layer].pop(0)
        sc = np.asarray(scores, dtype=np.float32)
        for e in range(self.E):
            hit = 1.0 if e in chosen else 0.0
            self.ema[layer][e] = self.lam * self.ema[layer][e] + (1.0 - self.lam) * hit
            self.score[layer][e] = float(sc[e])
            if hit:
                self.last[layer][e] = n

    def _features(self, layer: int):
        cnt = [float(sum(1 for s in self.sel[layer] if e in s)) for e in range(self.E)]
        age = [float(self.steps[layer] - self.last[layer][e]) for e in range(self.E)]
        return cnt, self.ema[layer], self.score[layer], age

    def keep(self, layer: int, expert: int) -> float:
        cnt, ema, score, age = self._features(layer)

        def norm(f, e):
            m = max(f)
            return f[e] / m if m > 0.0 else 0.0

        m_age = max(age)
        fresh = 1.0 - age[expert] / m_age if m_age > 0.0 else 1.0
        total = self.w[0] * norm(cnt, expert)
        total += self.w[1] * norm(ema, expert)
        total += self.w[2] * norm(score, expert)
        total += self.w[3] * fresh
        return total


class ScoredSlotPlanner(LruSlotPlanner):
    """The residency plan of LruSlotPlanner with the victims chosen by an
    eviction score ([HybriMoE] Minus Recent Score, [MoE-CORE] routing-history
    score): each call first records the step's routing scores, then the slots
    not holding a hit are taken by (owner's score, last use, slot id)
    ascending; empty slots still come first and everything else is unchanged.
    """

    def __init__(self, num_slots: int, layers: int, E: int, policy,
                 residency: list[tuple[int, int] | None] | None = None):
        super().__init__(num_slots, layers, E, residency)
        self.policy = policy
        self._victim_key = lambda s: (self.policy.keep(*self.owner[s]), self.last_use[s], s)

    def plan(self, layer: int, distinct, scores=None) -> list[Wave]:
        self.policy.observe(layer, scores, distinct)
        return super().plan(layer, distinct)


# ------------------------------------------------- split-precision experts ---
def round_bf16(a) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    u = np.ascontiguousarray(as_f32(a)).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def quantize_sym_g128(w, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric b-bit quantisation in groups of 128 along K of w [rows, K]:
    s = bf16(max|w_group| / (2^(b-1) - 1)), q = clip(rint(w / s), -2^(b-1), 2^(b-1) - 1),
    q = 0 where s = 0. The division and rounding that decide q are float32 (the
    4-bit rule of the int4 workload, widened to b bits for the residual split).
    Returns q int8 [rows, K] and s float32 [rows, K/128] (bf16 values)."""
    w32 = as_f32(w)
    rows, K = w32.shape
    g = w32.reshape(rows, K // 128, 128)
    qmax = np.float32(2 ** (bits - 1) - 1)
    s = round_bf16(np.max(np.abs(g), axis=2) / qmax)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s[:, :, None])
    q = np.where(s[:, :, None] == 0, 0, np.clip(q, -2 ** (bits - 1), 2 ** (bits - 1) - 1))
    return q.reshape(rows, K).astype(np.int8), s


def _deq(q, s) -> np.ndarray:
    return q.astype(np.float64) * np.repeat(s.astype(np.float64), 128, axis=1)


def resplit_expert(gate, up, down, bq: int = 4, br: int = 4) -> dict:
    """[RapidMoE] Algorithm 3 (RESplit): gate and up are quantised to b_q bits
    (W^Q) and their residual W - W^Q to b_r bits (W^R), so W^H = W^Q + W^R and
    W^L = W^Q; down is quantised twice, to b_q bits (W^L) and to b_q + b_r bits
    (W^H). The residual is formed in float32 from the float32 weights.
    Returns int8 code arrays and float32 (bf16-valued) scales per part."""
    out = {}
    for name, w in (("gate", gate), ("up", up)):
        q, s = quantize_sym_g128(w, bq)
        r = as_f32(w) - (q.astype(np.float32) * np.repeat(s, 128, axis=1))
        rq, rs = quantize_sym_g128(r, br)
        out[name + "_q"], out[name + "_s"], out[name + "_rq"], out[name + "_rs"] = q, s, rq, rs
    out["down_lq"], out["down_ls"] = quantize_sym_g128(down, bq)
    out["down_hq"], out["down_hs"] = quantize_sym_g128(down, bq + br)
    return out


def critical_threshold(theta: float, beta_l: float, phase: str, alpha: float) -> float:
    """[RapidMoE] Eqs. (3) and (5): Theta(l, t) = Theta * beta(l) * gamma(t), with
    gamma = 1 for prefill and alpha for decode."""
    gamma = {"prefill": 1.0, "decode": alpha}[phase]
    return theta * beta_l * gamma


def critical_experts(scores, distinct, threshold) -> list[int]:
    """[RapidMoE] Eq. (4) with Algorithm 1: the routed experts whose router score
    (softmax probability, averaged over the step's tokens for several tokens)
    is at least the threshold. The comparison is float32 (the kernels'), since
    it decides set membership."""
    sc = as_f32(scores)
    th = np.float32(threshold)
    return [int(e) for e in distinct if sc[int(e)] >= th]


def swiglu_expert_split(x_rows, w: dict, critical: bool) -> np.ndarray:
    """[RapidMoE] Algorithm 1 and Eq. (7): a critical expert runs on
    W^H (gate, up = W^Q + W^R; down = its b_q + b_r bit quantisation), any other
    routed expert on W^L (= W^Q; down at b_q bits). Activations are the int8
    rows of the int4 workload (x and the SwiGLU intermediate quantised per row);
    products in float64 on exactly dequantised weights."""
    qx, sx = quantize_rows_int8(x_rows)
    xh = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    def wg(name):
        W = _deq(w[name + "_q"], w[name + "_s"])
        return W + _deq(w[name + "_rq"], w[name + "_rs"]) if critical else W
    g = xh @ wg("gate").T
    u = xh @ wg("up").T
    with np.errstate(over="ignore"):
        h = silu(g) * u
    qh, sh = quantize_rows_int8(h.astype(np.float32))
    hh = qh.astype(np.float64) * sh.astype(np.float64)[:, None]
    down = _deq(w["down_hq"], w["down_hs"]) if critical else _deq(w["down_lq"], w["down_ls"])
    return hh @ down.T


# ------------------------------------------------------------- full layer ---
def moe_layer(x, w_router, bias, k: int, *, layer: int, pool: SlotPool,
              planner: LruSlotPlanner | None, weights_of_expert,
              shared: list[dict] | None = None, renorm: bool = True,
              scores=None, critical=None, rows=None) -> dict:
    """One routed-expert layer over the slot pool.

    route -> permute -> residency plan -> for each wave of the plan: the
    wave's fills copy the expert's weights into their slots (the slot's
    previous expert leaves the table), then each (t, j) routed to an expert
    the wave computes runs with the weights read through pool.lut as it stands
    after those fills -> weighted combine (+ shared experts, weight 1).
    A later wave may overwrite a slot an earlier wave read; the earlier
    experts are already computed ([SeqMoE] Mechanism: the expert kernel reads
    experts through the slot table; misses are copied in before use).
    Without a planner every routed expert must already be resident.
    ``weights_of_expert(e)`` returns the host-store weights of expert e of
    this layer (what a fill copies).

    scores: the step's routing scores, handed to a scored planner's plan.
    critical: for split-precision weights, the routed experts that run at high
    precision ([RapidMoE] Algorithm 1; None = all); shared experts always do.
    rows: token indices whose outputs are computed (None = all); the routing,
    the permutation and the plan still cover every token, and the other rows
    of ``y`` and ``out`` stay zero.
    """
    r = route(x, w_router, bias, k, renorm)
    ids = r["ids"]
    p = permute(ids, w_router.shape[0])
    if planner is not None:
        waves = (planner.plan(layer, p["distinct"]) if scores is None
                 else planner.plan(layer, p["distinct"], scores))
    else:
        waves = [Wave(compute=[int(e) for e in p["distinct"]])]
    x_rows = as_f32(x)  # exact for fp32 and bf16 tokens; each expert form converts further
    T = ids.shape[0]
    H = as_f64(w_router).shape[1]
    keep = np.ones(T, dtype=bool) if rows is None else np.isin(np.arange(T), rows)
    y = np.zeros((T, k, H), dtype=np.float64)
    for wave in waves:
        for e, s in wave.fills:
            pool.commit(s, layer, e, weights_of_expert(e))
        for e in wave.compute:
            e = int(e)
            f = p["perm"][p["offsets"][e]:p["offsets"][e + 1]]
            f = f[keep[f // k]]
            if f.size == 0:
                continue
            t_rows, j_rows = f // k, f % k
            hi = critical is None or e in critical
            y[t_rows, j_rows] = expert_forward(x_rows[t_rows], pool.weights_of(layer, e), hi)
    if planner is not None and not np.array_equal(pool.lut, planner.lut):
        raise AssertionError("pool table differs from the planner's after the last wave")
    sel = np.flatnonzero(keep)
    y_sh = []
    for w in shared or []:
        ys = np.zeros((T, H), dtype=np.float64)
        ys[sel] = expert_forward(x_rows[sel], w, True)
        y_sh.append(ys)
    out = combine(y, r["weights"], y_sh)
    out[~keep] = 0.0
    return dict(route=r, perm=p, waves=waves if planner is not None else [], y=y,
                y_shared=y_sh, out=out)
