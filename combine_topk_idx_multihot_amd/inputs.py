"""Seeded synthetic workloads for the MoE dispatch/combine path.

This module only draws inputs: router logits, top-k expert ids, routing weights
and bf16 activations.  It holds none of the dispatch/combine arithmetic and
imports neither the GPU library nor the oracle, so both sides can be fed the
same arrays.

Layer shapes follow the benchmark section of "Add the deepep expert-parallel
implementation" (a Qwen3-30B-A3B-shaped layer, E=128, H=2048, top-8, and an
H=4096 layer, E=128, top-8); ids of -1 mark empty slots as in the multihot
conversion of "feat: add hybridep".  The router itself is not part of the path:
top-k of a softmax is drawn here on the CPU.

Recipe (every stream comes from ``SeedSequence(seed).spawn``):
  * logits: N(0,1) float32 [T,E]; top-k = experts sorted by descending logit,
    the lower id first on ties (softmax is monotone, so this is top-k of the
    softmax); weights = softmax over the chosen logits, renormalised in fp32.
  * skewed routing: k experts drawn without replacement with probability
    proportional to (e+1)^-alpha (Gumbel-top-k on -alpha*ln(e+1)); weights
    as above from independent N(0,1) logits over the drawn experts; then a
    fraction of slots set to -1 and a fraction of tokens set all -1.
  * bf16 tensors: N(0,1) float32 rounded to bf16 (nearest-even, via torch on
    the CPU) and returned as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAMS = ("logits", "hidden", "grad", "expert_out", "masks", "weights")


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    lb: int = 0
    EL: int | None = None      # None -> all E experts local
    P: int = 1                 # pad_multiple
    sync_free: bool = False
    capacity: int | None = None  # sync-free rows; None -> T*min(k,EL) + EL*(P-1)
    skew_alpha: float | None = None
    invalid_slot_frac: float = 0.0
    invalid_token_frac: float = 0.0
    backward: bool = False
    note: str = ""

    @property
    def num_local(self) -> int:
        return self.E if self.EL is None else self.EL

    @property
    def cap(self) -> int:
        if self.capacity is not None:
            return self.capacity
        EL = self.num_local
        return self.T * min(self.k, EL) + EL * (self.P - 1)


# The five workloads of the benchmark description.
WORKLOADS = {
    "tiny": Workload("tiny", T=256, H=256, E=8, k=2, P=1,
                     note="tiny dispatch+combine, eager"),
    "qwen3_30b_a3b": Workload("qwen3_30b_a3b", T=4096, H=2048, E=128, k=8, P=16,
                              note="Qwen3-30B-A3B-shaped layer, eager"),
    "h4096_rank_share": Workload("h4096_rank_share", T=16384, H=4096, E=128, k=8, lb=0, EL=16,
                                 P=1, sync_free=True, capacity=16384 * 8,
                                 note="H=4096 layer, one rank's share (experts 0..15), "
                                      "sync-free worst-case capacity T*8"),
    "skewed": Workload("skewed", T=8192, H=2048, E=128, k=8, P=128, skew_alpha=1.2,
                       invalid_slot_frac=0.10, invalid_token_frac=0.01,
                       note="Zipf(1.2) routing, 10% slots -1, 1% tokens all -1, eager"),
    "backward_h4096": Workload("backward_h4096", T=16384, H=4096, E=128, k=8, P=16,
                               backward=True,
                               note="combine_bwd (cached dispatch + dw) at T=16384, H=4096"),
}


def _streams(seed: int) -> dict:
    ss = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.default_rng(s) for name, s in zip(STREAMS, ss)}


def _softmax_renorm(logits_sel: np.ndarray) -> np.ndarray:
    """fp32 softmax over the chosen experts' logits (rows), i.e. the full
    softmax restricted to the chosen experts and renormalised."""
    z = logits_sel.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z, dtype=np.float32)
    return (p / p.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def topk_softmax(T: int, E: int, k: int, rng: np.random.Generator):
    """Top-k expert ids (distinct) and fp32 weights from N(0,1) router logits."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    return order.astype(np.int32), _softmax_renorm(sel)


def topk_zipf(T: int, E: int, k: int, alpha: float, rng: np.random.Generator,
              wrng: np.random.Generator):
    """k distinct experts per token drawn without replacement with
    P(e) proportional to (e+1)^-alpha (Gumbel-top-k)."""
    base = (-alpha * np.log(np.arange(1, E + 1, dtype=np.float64)))[None, :]
    g = rng.gumbel(size=(T, E))
    order = np.argsort(-(base + g), axis=1, kind="stable")[:, :k]
    lw = wrng.standard_normal((T, k), dtype=np.float32)
    return order.astype(np.int32), _softmax_renorm(lw)


def bf16_normal(shape, rng: np.random.Generator) -> np.ndarray:
    """N(0,1) values rounded to bf16; returned as uint16 bit patterns."""
    import torch

    a = rng.standard_normal(shape, dtype=np.float32)
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Case:
    wl: Workload
    seed: int
    idx: np.ndarray            # [T,k] int32
    w: np.ndarray              # [T,k] float32
    x: np.ndarray | None = None        # [T,H] uint16 (bf16 bits)
    grad_out: np.ndarray | None = None  # [T,H] uint16
    extra: dict = field(default_factory=dict)


def make_routing(wl: Workload, seed: int):
    s = _streams(seed)
    if wl.skew_alpha is not None:
        idx, w = topk_zipf(wl.T, wl.E, wl.k, wl.skew_alpha, s["logits"], s["weights"])
    else:
        idx, w = topk_softmax(wl.T, wl.E, wl.k, s["logits"])
    if wl.invalid_slot_frac > 0:
        drop = s["masks"].random((wl.T, wl.k)) < wl.invalid_slot_frac
        idx[drop] = -1
    if wl.invalid_token_frac > 0:
        dead = s["masks"].random(wl.T) < wl.invalid_token_frac
        idx[dead, :] = -1
    return idx, w


def make_case(wl: Workload | str, seed: int | None = None, hidden: bool = True,
              grad: bool = False) -> Case:
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if seed is None:
        seed = 1000 + list(WORKLOADS).index(wl.name) + 1 if wl.name in WORKLOADS else 1000
    idx, w = make_routing(wl, seed)
    s = _streams(seed)
    x = bf16_normal((wl.T, wl.H), s["hidden"]) if hidden else None
    g = bf16_normal((wl.T, wl.H), s["grad"]) if grad else None
    return Case(wl=wl, seed=seed, idx=idx, w=w, x=x, grad_out=g)


def expert_out_rows(R: int, H: int, seed: int) -> np.ndarray:
    """Stand-in for the experts' output rows (before the routing weight): bf16 N(0,1)."""
    return bf16_normal((R, H), _streams(seed)["expert_out"])


def random_routing(T: int, E: int, k: int, rng: np.random.Generator, p_invalid: float = 0.0,
                   p_out_of_range: float = 0.0, allow_dup: bool = False) -> np.ndarray:
    """Edge-case routing for tests: uniform ids, optional -1 slots, optional
    repeated ids inside a token, optional ids outside [-1, E)."""
    if allow_dup:
        idx = rng.integers(0, E, size=(T, k))
    else:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
    idx = idx.astype(np.int64)
    if p_invalid > 0:
        idx[rng.random((T, k)) < p_invalid] = -1
    if p_out_of_range > 0:
        bad = rng.random((T, k)) < p_out_of_range
        vals = rng.choice(np.array([-7, -2, E, E + 5, 1 << 20]), size=(T, k))
        idx[bad] = vals[bad]
    return idx
