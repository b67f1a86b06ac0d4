"""Input preparation in front of the recurrence, in float64: L2 normalisation of q and k
and the gate activations that turn pre-activation inputs into alpha, erase and write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source. The course page "GDN, KDA và Mamba-2 · cập nhật state trong hybrid", section 2,
puts "project and prepare q/k/v" as the step in front of "decay, then correct the
state". The pages do not spell out that preparation; the workloads the method is
measured on fix it: q and k are L2-normalised per token and head; the KDA decay is
alpha = exp(-c * softplus(z)) channel-wise (c = 1, or c = 0.1 for the long-memory
setting); Complex KDA's decay is alpha = tanh(z) in [-1, 1]; beta, e and w are
sigmoid(z), and Complex KDA's beta is 2 sigmoid(z) in [0, 2]. Readings taken:
  * L2 normalisation is x / ||x||_2 over d_k, with a zero vector left at zero (no
    epsilon is added).
  * softplus(z) = log(1 + e^z); sigmoid(z) = 1 / (1 + e^-z); both evaluated in a
    form that does not overflow, with sigmoid(+inf) = 1, sigmoid(-inf) = 0,
    tanh(+-inf) = +-1, exp(-c * softplus(-inf)) = 1.
"""
from __future__ import annotations

import numpy as np

from .recurrence import _f64

ALPHA_ACTS = ("none", "exp_neg_softplus", "tanh")
GATE_ACTS = ("none", "sigmoid")


def l2_normalize(x):
    """x / ||x|| over the last axis; zero vectors stay zero.

    Pinned by: unit norm of the result, invariance to positive scaling of x, the
    zero vector, and a hand example ((3, 4) -> (0.6, 0.8))."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def softplus(z):
    """log(1 + e^z) without overflow. Pinned by softplus(0) = log 2 and the large-|z|
    asymptotes softplus(z) -> z, softplus(-z) -> e^-z."""
    return np.logaddexp(0.0, _f64(z))


def sigmoid(z):
    """1 / (1 + e^-z) without overflow. Pinned by sigmoid(0) = 1/2, sigmoid(z) +
    sigmoid(-z) = 1 and the limits at +-inf."""
    z = _f64(z)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def alpha_from(z, act: str, scale: float = 1.0):
    """Decay gate from its pre-activation: ``none`` passes z through; ``exp_neg_softplus``
    gives exp(-scale * softplus(z)) in (0, 1]; ``tanh`` gives tanh(z) in [-1, 1].

    Pinned by: softplus(0) = log 2, so z = 0 gives 2^-scale; z = -inf gives exactly 1;
    exp(-softplus(z)) = sigmoid(-z) at scale 1; tanh(+-inf) = +-1, tanh is odd, the exact
    values tanh(ln x) = (x^2 - 1) / (x^2 + 1) (e.g. tanh(ln 2) = 3/5), its series near zero
    and 1 - tanh z = 2 e^{-2z} / (1 + e^{-2z})."""
    z = _f64(z)
    if act == "none":
        return z
    if act == "exp_neg_softplus":
        return np.exp(-scale * softplus(z))
    if act == "tanh":
        return np.tanh(z)
    raise ValueError(f"unknown decay activation {act!r}")


def gate_from(z, act: str, scale: float = 1.0):
    """Erase or write gate from its pre-activation: ``none`` passes z through,
    ``sigmoid`` gives scale * sigmoid(z) (scale 2 gives Complex KDA's beta in [0, 2]).

    Pinned by sigmoid's values at 0 and +-inf, its symmetry and the exact values
    sigmoid(+-ln x) = x / (x + 1), 1 / (x + 1) (e.g. sigmoid(ln 3) = 3/4)."""
    z = _f64(z)
    if z is None:
        return None
    if act == "none":
        return z
    if act == "sigmoid":
        return scale * sigmoid(z)
    raise ValueError(f"unknown gate activation {act!r}")


def prepare(q, k, alpha_z, erase_z, write_z, *, l2norm_qk: bool, alpha_act: str, alpha_scale: float,
            gate_act: str, gate_scale: float):
    """The prepared inputs (q, k, alpha, erase, write) the recurrence consumes.

    Pinned through its parts (above) and by: with every option off it returns its
    inputs unchanged; the recurrence on prepared inputs is unchanged when q and k are
    scaled by positive factors before normalisation."""
    q, k = _f64(q), _f64(k)
    if l2norm_qk:
        q, k = l2_normalize(q), l2_normalize(k)
    alpha = alpha_from(alpha_z, alpha_act, alpha_scale)
    erase = gate_from(erase_z, gate_act, gate_scale)
    write = None if write_z is None else gate_from(write_z, gate_act, gate_scale)
    return q, k, alpha, erase, write
