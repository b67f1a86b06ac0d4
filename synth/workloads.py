"""Seeded synthetic workloads for the gated delta-rule recurrence.

Every array is drawn in float64 from a numpy PCG64 generator, in a fixed
order (q, k, v, alpha noise, erase noise, write noise, initial state, masks),
then rounded to float32 and, for bf16 workloads, to the nearest bfloat16
(round to nearest, ties to even). The rounded values are kept in float32
arrays, so a bf16 tensor built from them is exact and an fp64 upcast of them
is exactly what the GPU receives.

Gate recipes follow the workload descriptions: channel-wise decay alpha per
key channel, per-head scalar erase/write gates (KDA, RDA), channel-wise
erase on the key and write on the value (GDN-2), and the Complex KDA ranges
(alpha in [-1, 1], beta in [0, 2]).  The notation is that of the update rules
in the Raon-1-mini-preview discussion (Hugging Face, discussion #1) and of
the Complex KDA abstract (arXiv 2609.24797).

No part of the recurrence is computed here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

VARIANTS = ("kda", "rda", "gdn2", "ckda")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def _to_input(x64: np.ndarray, in_dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if in_dtype == "bf16":
        return bf16_round(x32)
    if in_dtype == "f32":
        return x32
    raise ValueError(f"unknown input dtype {in_dtype!r}")


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-300)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


# Gate recipes: each turns standard-normal noise into gate values.
#   "kda_tiny": alpha = exp(-softplus(z)) in (0, 1), beta = sigmoid(z)
#   "kda":      alpha = exp(-0.1 softplus(z)) (about 0.9 .. 1), beta = sigmoid(z)
#   "rda":      alpha as "kda"; erase e and write w independent per-head sigmoids
#   "gdn2":     alpha as "kda"; erase b in R^dk and write w in R^dv, channel-wise sigmoids
#   "ckda":     alpha = tanh(1.5 z) in [-1, 1] with about 10% of entries forced to +-1,
#               beta = 2 sigmoid(z) in [0, 2] with about 5% of token-heads at exactly 2
RECIPES = ("kda_tiny", "kda", "rda", "gdn2", "ckda")


def recipe_variant(recipe: str) -> str:
    return {"kda_tiny": "kda", "kda": "kda", "rda": "rda", "gdn2": "gdn2", "ckda": "ckda"}[recipe]


@dataclass
class Workload:
    """One input set. Prefill layout: q,k [B,T,H,dk]; v [B,T,H,dv]; alpha [B,T,H,dk];
    erase [B,T,H] (or [B,T,H,dk] for GDN-2); write None (KDA/CKDA), [B,T,H] (RDA) or
    [B,T,H,dv] (GDN-2); S0 [N,H,dk,dv] or None (zero state); cu_seqlens [N+1] int32 or
    None. Decode layout drops the T axis and uses N for the batch of sequences."""

    name: str
    variant: str
    in_dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    erase: np.ndarray
    write: Optional[np.ndarray]
    S0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray] = None
    chunk: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        if self.cu_seqlens is not None:
            return len(self.cu_seqlens) - 1
        return self.q.shape[0]


def _draw_gates(rng, recipe: str, lead: tuple, dk: int, dv: int):
    """Draw alpha, erase, write in the fixed order alpha, erase, write, then masks."""
    za = rng.standard_normal(lead + (dk,))
    if recipe == "gdn2":
        ze = rng.standard_normal(lead + (dk,))
        zw = rng.standard_normal(lead + (dv,))
    elif recipe == "rda":
        ze = rng.standard_normal(lead)
        zw = rng.standard_normal(lead)
    else:
        ze = rng.standard_normal(lead)
        zw = None
    return za, ze, zw


def _finish_gates(rng, recipe: str, za, ze, zw, masks_rng=None):
    if recipe == "kda_tiny":
        alpha = np.exp(-_softplus(za))
    elif recipe == "ckda":
        alpha = np.tanh(1.5 * za)
    else:
        alpha = np.exp(-0.1 * _softplus(za))
    if recipe in ("kda_tiny", "kda"):
        erase, write = _sigmoid(ze), None
    elif recipe == "ckda":
        erase, write = 2.0 * _sigmoid(ze), None
    else:
        erase, write = _sigmoid(ze), _sigmoid(zw)
    return alpha, erase, write


def _ckda_masks(rng, alpha, erase):
    force = rng.random(alpha.shape) < 0.10
    sign = np.where(rng.random(alpha.shape) < 0.5, -1.0, 1.0)
    alpha = np.where(force, sign, alpha)
    at_two = rng.random(erase.shape) < 0.05
    erase = np.where(at_two, 2.0, erase)
    return alpha, erase


# Pre-activation form of each recipe, for the fused input preparation: the decay and gate
# activations (and q/k normalisation) are then applied by the consumer, not here.
#   alpha_act/alpha_scale: "exp_neg_softplus" with c = 1 (kda_tiny) or 0.1, or "tanh" (ckda,
#   whose pre-activation is 1.5 z); gate_act "sigmoid" with scale 1, or 2 for ckda's beta.
PREP = {
    "kda_tiny": dict(l2norm_qk=True, alpha_act="exp_neg_softplus", alpha_scale=1.0, gate_act="sigmoid", gate_scale=1.0),
    "kda": dict(l2norm_qk=True, alpha_act="exp_neg_softplus", alpha_scale=0.1, gate_act="sigmoid", gate_scale=1.0),
    "rda": dict(l2norm_qk=True, alpha_act="exp_neg_softplus", alpha_scale=0.1, gate_act="sigmoid", gate_scale=1.0),
    "gdn2": dict(l2norm_qk=True, alpha_act="exp_neg_softplus", alpha_scale=0.1, gate_act="sigmoid", gate_scale=1.0),
    "ckda": dict(l2norm_qk=True, alpha_act="tanh", alpha_scale=1.0, gate_act="sigmoid", gate_scale=2.0),
}


def _preact_gates(rng, recipe: str, za, ze, zw):
    """Pre-activations in the draw order of the activated recipe: Complex KDA's forced
    decays become +-inf (tanh -> +-1) and its beta = 2 entries +inf (2 sigmoid -> 2)."""
    if recipe == "ckda":
        za = 1.5 * za
        force = rng.random(za.shape) < 0.10
        sign = np.where(rng.random(za.shape) < 0.5, -1.0, 1.0)
        za = np.where(force, sign * np.inf, za)
        at_two = rng.random(ze.shape) < 0.05
        ze = np.where(at_two, np.inf, ze)
    return za, ze, zw


def draw_varlen_lengths(rng, n: int = 12, total: int = 32768, lo: int = 256, hi: int = 6000):
    """Draw n-1 lengths uniformly (integers in [lo, hi]) and set the last so the lengths
    sum to total; redraw until the last one also lies in [lo, hi]."""
    if n * lo > total or n * hi < total:
        raise ValueError("no length vector satisfies the constraints")
    for _ in range(100000):
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)
    raise RuntimeError("length draw did not converge")


def make_prefill(recipe: str, B: int, T: int, H: int, dk: int, dv: int, *,
                 in_dtype: str = "bf16", seed: int = 0, random_s0: bool = True,
                 lengths=None, chunk: int = 64, name: str = "", preact: bool = False,
                 alpha_dtype: str = "f32") -> Workload:
    """Prefill workload. With ``lengths`` the sequences are packed along T of a single
    batch row (B must be 1) and described by cu_seqlens. With ``preact`` q and k are not
    normalised and alpha / erase / write hold pre-activations (``meta["prep"]`` names the
    activations); ``alpha_dtype="bf16"`` rounds alpha to bfloat16."""
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(cu) - 1 if cu is not None else B
    lead = (B, T, H)
    q, k = rng.standard_normal(lead + (dk,)), rng.standard_normal(lead + (dk,))
    if not preact:
        q, k = _l2_normalise(q), _l2_normalise(k)
    v = rng.standard_normal(lead + (dv,))
    za, ze, zw = _draw_gates(rng, recipe, lead, dk, dv)
    S0 = rng.standard_normal((N, H, dk, dv)) / np.sqrt(dk) if random_s0 else None
    if preact:
        alpha, erase, write = _preact_gates(rng, recipe, za, ze, zw)
    else:
        alpha, erase, write = _finish_gates(rng, recipe, za, ze, zw)
        if recipe == "ckda":
            alpha, erase = _ckda_masks(rng, alpha, erase)
    meta = {"recipe": recipe, "seed": seed, "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
            "lengths": None if lengths is None else [int(x) for x in lengths]}
    if preact:
        meta["prep"] = dict(PREP[recipe], alpha_dtype=alpha_dtype)
    return Workload(
        name=name or f"{recipe}_B{B}_T{T}_H{H}_d{dk}x{dv}" + ("_preact" if preact else ""),
        variant=recipe_variant(recipe), in_dtype=in_dtype,
        q=_to_input(q, in_dtype), k=_to_input(k, in_dtype), v=_to_input(v, in_dtype),
        alpha=_to_input(alpha, alpha_dtype), erase=erase.astype(np.float32),
        write=None if write is None else write.astype(np.float32),
        S0=None if S0 is None else S0.astype(np.float32), cu_seqlens=cu, chunk=chunk, meta=meta,
    )


def make_decode(recipe: str, N: int, H: int, dk: int, dv: int, *, steps: int = 1,
                in_dtype: str = "bf16", seed: int = 0, with_state: bool = True,
                name: str = "", preact: bool = False, alpha_dtype: str = "f32") -> Workload:
    """Decode workload: ``steps`` consecutive single-token inputs for N sequences x H heads.
    Token arrays have a leading step axis: q,k [steps,N,H,dk], v [steps,N,H,dv], gates
    likewise. S0 [N,H,dk,dv] is the state before the first step."""
    rng = np.random.default_rng(seed)
    lead = (steps, N, H)
    q, k = rng.standard_normal(lead + (dk,)), rng.standard_normal(lead + (dk,))
    if not preact:
        q, k = _l2_normalise(q), _l2_normalise(k)
    v = rng.standard_normal(lead + (dv,))
    za, ze, zw = _draw_gates(rng, recipe, lead, dk, dv)
    S0 = None
    if with_state:
        S0 = (rng.standard_normal((N, H, dk, dv)) / np.sqrt(dk)).astype(np.float32)
    if preact:
        alpha, erase, write = _preact_gates(rng, recipe, za, ze, zw)
    else:
        alpha, erase, write = _finish_gates(rng, recipe, za, ze, zw)
        if recipe == "ckda":
            alpha, erase = _ckda_masks(rng, alpha, erase)
    meta = {"recipe": recipe, "seed": seed, "N": N, "H": H, "dk": dk, "dv": dv, "steps": steps}
    if preact:
        meta["prep"] = dict(PREP[recipe], alpha_dtype=alpha_dtype)
    return Workload(
        name=name or f"decode_{recipe}_N{N}_H{H}_d{dk}x{dv}_s{steps}" + ("_preact" if preact else ""),
        variant=recipe_variant(recipe), in_dtype=in_dtype,
        q=_to_input(q, in_dtype), k=_to_input(k, in_dtype), v=_to_input(v, in_dtype),
        alpha=_to_input(alpha, alpha_dtype), erase=erase.astype(np.float32),
        write=None if write is None else write.astype(np.float32),
        S0=S0, cu_seqlens=None, chunk=1, meta=meta,
    )


def _product_draw(rng, recipe: str, lead: tuple, dk: int, dv: int, preact: bool):
    """q, k (two keys per token), v (two values), alpha, beta (two) in that draw order."""
    if recipe not in ("kda", "ckda"):
        raise ValueError("two-transition workloads use the kda or ckda gate recipe")
    q = rng.standard_normal(lead + (dk,))
    k = rng.standard_normal(lead + (2, dk))
    if not preact:
        q, k = _l2_normalise(q), _l2_normalise(k)
    v = rng.standard_normal(lead + (2, dv))
    za = rng.standard_normal(lead + (dk,))
    zb = rng.standard_normal(lead + (2,))
    if preact:
        alpha, beta, _ = _preact_gates(rng, recipe, za, zb, None)
    else:
        alpha, beta, _ = _finish_gates(rng, recipe, za, zb, None)
        if recipe == "ckda":
            alpha, beta = _ckda_masks(rng, alpha, beta)
    return q, k, v, alpha, beta


def make_product(recipe: str, B: int, T: int, H: int, dk: int, dv: int, *, in_dtype: str = "bf16",
                 seed: int = 0, random_s0: bool = True, lengths=None, name: str = "", preact: bool = False,
                 alpha_dtype: str = "f32") -> Workload:
    """Prefill workload of the two-transitions-per-token variant: q, alpha [B,T,H,dk];
    k [B,T,H,2,dk] (each key L2-normalised); v [B,T,H,2,dv]; erase = beta [B,T,H,2] with the
    gate recipe's distribution for each transition; write None. ``lengths`` packs as in
    ``make_prefill``."""
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(cu) - 1 if cu is not None else B
    q, k, v, alpha, beta = _product_draw(rng, recipe, (B, T, H), dk, dv, preact)
    S0 = rng.standard_normal((N, H, dk, dv)) / np.sqrt(dk) if random_s0 else None
    meta = {"recipe": recipe, "seed": seed, "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "transitions": 2,
            "lengths": None if lengths is None else [int(x) for x in lengths]}
    if preact:
        meta["prep"] = dict(PREP[recipe], alpha_dtype=alpha_dtype)
    return Workload(
        name=name or f"product2_{recipe}_B{B}_T{T}_H{H}_d{dk}x{dv}" + ("_preact" if preact else ""),
        variant="product2", in_dtype=in_dtype,
        q=_to_input(q, in_dtype), k=_to_input(k, in_dtype), v=_to_input(v, in_dtype),
        alpha=_to_input(alpha, alpha_dtype), erase=beta.astype(np.float32), write=None,
        S0=None if S0 is None else S0.astype(np.float32), cu_seqlens=cu, chunk=64, meta=meta,
    )


def make_product_decode(recipe: str, N: int, H: int, dk: int, dv: int, *, steps: int = 1,
                        in_dtype: str = "bf16", seed: int = 0, name: str = "", preact: bool = False,
                        alpha_dtype: str = "f32") -> Workload:
    """Decode workload of the two-transitions-per-token variant: q, alpha [steps,N,H,dk];
    k [steps,N,H,2,dk]; v [steps,N,H,2,dv]; beta [steps,N,H,2]; S0 [N,H,dk,dv]."""
    rng = np.random.default_rng(seed)
    q, k, v, alpha, beta = _product_draw(rng, recipe, (steps, N, H), dk, dv, preact)
    S0 = (rng.standard_normal((N, H, dk, dv)) / np.sqrt(dk)).astype(np.float32)
    meta = {"recipe": recipe, "seed": seed, "N": N, "H": H, "dk": dk, "dv": dv, "steps": steps, "transitions": 2}
    if preact:
        meta["prep"] = dict(PREP[recipe], alpha_dtype=alpha_dtype)
    return Workload(
        name=name or f"decode_product2_{recipe}_N{N}_H{H}_d{dk}x{dv}_s{steps}",
        variant="product2", in_dtype=in_dtype,
        q=_to_input(q, in_dtype), k=_to_input(k, in_dtype), v=_to_input(v, in_dtype),
        alpha=_to_input(alpha, alpha_dtype), erase=beta.astype(np.float32), write=None,
        S0=S0, cu_seqlens=None, chunk=1, meta=meta,
    )


# The five workloads the path is measured and checked on.  Seeds are 1000 + the
# workload number (1-based).
PRESETS = {
    # 1: KDA, fp32 inputs, B=1 H=2 T=64 d=16, chunk 16, zero initial state
    "kda_tiny": dict(kind="prefill", recipe="kda_tiny", B=1, T=64, H=2, dk=16, dv=16,
                     in_dtype="f32", seed=1001, random_s0=False, chunk=16),
    # 2: KDA prefill, bf16, B=4 H=16 T=4096 d=128, chunk 64, random fp32 S0
    "kda_prefill": dict(kind="prefill", recipe="kda", B=4, T=4096, H=16, dk=128, dv=128,
                        in_dtype="bf16", seed=1002, random_s0=True, chunk=64),
    # 3: RDA and GDN-2 varlen, 12 packed sequences, 32768 tokens, H=16 d=128, bf16
    "rda_varlen": dict(kind="varlen", recipe="rda", total=32768, nseq=12, lo=256, hi=6000,
                       H=16, dk=128, dv=128, in_dtype="bf16", seed=1003, chunk=64),
    "gdn2_varlen": dict(kind="varlen", recipe="gdn2", total=32768, nseq=12, lo=256, hi=6000,
                        H=16, dk=128, dv=128, in_dtype="bf16", seed=1003, chunk=64),
    # 4: Complex KDA long context, B=2 H=16 T=16384 d=128, bf16
    "ckda_long": dict(kind="prefill", recipe="ckda", B=2, T=16384, H=16, dk=128, dv=128,
                      in_dtype="bf16", seed=1004, random_s0=True, chunk=64),
    # 5: decode, 512 sequences x 32 heads, d=128, every variant
    "decode_kda": dict(kind="decode", recipe="kda", N=512, H=32, dk=128, dv=128,
                       in_dtype="bf16", seed=1005),
    "decode_rda": dict(kind="decode", recipe="rda", N=512, H=32, dk=128, dv=128,
                       in_dtype="bf16", seed=1005),
    "decode_gdn2": dict(kind="decode", recipe="gdn2", N=512, H=32, dk=128, dv=128,
                        in_dtype="bf16", seed=1005),
    "decode_ckda": dict(kind="decode", recipe="ckda", N=512, H=32, dk=128, dv=128,
                        in_dtype="bf16", seed=1005),
    # the two-transitions-per-token variant at the KDA prefill and decode shapes
    "product2_prefill": dict(kind="product", recipe="kda", B=4, T=4096, H=16, dk=128, dv=128,
                             in_dtype="bf16", seed=1006, random_s0=True),
    "decode_product2": dict(kind="product_decode", recipe="kda", N=512, H=32, dk=128, dv=128,
                            in_dtype="bf16", seed=1006),
}


def preset(name: str, **override) -> Workload:
    """Build a named workload; keyword overrides shrink it for quick checks."""
    p = dict(PRESETS[name])
    p.update(override)
    kind = p.pop("kind")
    if kind == "prefill":
        return make_prefill(p.pop("recipe"), p.pop("B"), p.pop("T"), p.pop("H"), p.pop("dk"),
                            p.pop("dv"), name=name, **p)
    if kind == "varlen":
        seed = p.pop("seed")
        lengths = draw_varlen_lengths(np.random.default_rng(seed), p.pop("nseq"), p.pop("total"),
                                      p.pop("lo"), p.pop("hi"))
        return make_prefill(p.pop("recipe"), 1, 0, p.pop("H"), p.pop("dk"), p.pop("dv"),
                            seed=seed + 7919, lengths=lengths, name=name, **p)
    if kind == "decode":
        return make_decode(p.pop("recipe"), p.pop("N"), p.pop("H"), p.pop("dk"), p.pop("dv"),
                           name=name, **p)
    if kind == "product":
        return make_product(p.pop("recipe"), p.pop("B"), p.pop("T"), p.pop("H"), p.pop("dk"),
                            p.pop("dv"), name=name, **p)
    if kind == "product_decode":
        return make_product_decode(p.pop("recipe"), p.pop("N"), p.pop("H"), p.pop("dk"), p.pop("dv"),
                                   name=name, **p)
    raise ValueError(kind)
