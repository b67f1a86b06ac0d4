"""Planted mistakes in the fp64 oracle, used by ``test_oracle_mutants.py``.

Loaded as a pytest plugin in a child process (``-p oracle_mutants`` with ``DR_ORACLE_MUTANT``
naming one entry of ``MUTANTS``), it rewrites one statement of one oracle function before the
pins are collected: the function's source is taken, the statement replaced and the new function
bound wherever the oracle package held the original. Each entry is a mistake that a plain
reading of the pages could plausibly make; the pins must catch every one of them. Nothing here
runs in the library or on a GPU.
"""
import importlib
import inspect
import os
import sys
import textwrap

# name -> (oracle module, function, statement as written in the oracle, planted replacement)
MUTANTS = {
    # the step rule (Hugging Face discussion "KRAFTON/Raon-1-mini-preview" #1, the three state updates)
    "write term dropped": ("recurrence", "step",
                           "S_new = erased + k[..., :, None] * m[..., None, :]", "S_new = erased"),
    "erase added, not subtracted": ("recurrence", "step", "erased = X - k[..., :, None]", "erased = X + k[..., :, None]"),
    "erase before decay": ("recurrence", "step",
                           'erased = X - k[..., :, None] * np.einsum("...i,...ij->...j", u, X)[..., None, :]',
                           'erased = alpha[..., :, None] * (S - k[..., :, None] * np.einsum("...i,...ij->...j", u, S)'
                           '[..., None, :])'),
    "readout before the update": ("recurrence", "step", 'o = np.einsum("...ij,...i->...j", S_new, q)',
                                  'o = np.einsum("...ij,...i->...j", S, q)'),
    "readout scaled by 1/sqrt(d_k)": ("recurrence", "step", 'o = np.einsum("...ij,...i->...j", S_new, q)',
                                      'o = np.einsum("...ij,...i->...j", S_new, q) / np.sqrt(q.shape[-1])'),
    "GDN-2 b on the left factor": ("recurrence", "step",
                                   'erased = X - k[..., :, None] * np.einsum("...i,...ij->...j", u, X)[..., None, :]',
                                   'erased = X - (u if variant == "gdn2" else k)[..., :, None] * np.einsum('
                                   '"...i,...ij->...j", k if variant == "gdn2" else u, X)[..., None, :]'),
    "RDA gates swapped": ("recurrence", "erase_write_vectors",
                          "u = erase[..., None] * k\n        m = write[..., None] * v",
                          "u = write[..., None] * k\n        m = erase[..., None] * v"),
    "GDN-2 erase gate averaged": ("recurrence", "erase_write_vectors", "u = erase * k",
                                  "u = erase.mean(axis=-1, keepdims=True) * k"),
    "packed sequences share a state": ("recurrence", "step_recurrence",
                                       "S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()",
                                       "S = (np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()) if n == 0 else S"),
    # the chunked form (unrolled step rule)
    "chunk ratio off by one token": ("chunked", "_chunk", "ratio[:, r, s] = ratio[:, r - 1, s] * alpha[:, r]",
                                     "ratio[:, r, s] = ratio[:, r - 1, s] * alpha[:, r - 1]"),
    "P without its diagonal": ("chunked", "_chunk",
                               'P = np.einsum("hri,hsi,hrsi->hrs", q, k, ratio) * np.tril(np.ones((L, L)), 0)',
                               'P = np.einsum("hri,hsi,hrsi->hrs", q, k, ratio) * np.tril(np.ones((L, L)), -1)'),
    "T from (I - A)": ("chunked", "_chunk", "np.linalg.solve(np.eye(L)[None] + A, rhs)",
                       "np.linalg.solve(np.eye(L)[None] - A, rhs)"),
    "Gamma exclusive of the token's own gate": ("chunked", "_chunk", "gamma = np.cumprod(alpha, axis=1)",
                                                "gamma = np.cumprod(alpha, axis=1) / alpha"),
    "Kbar decayed over the whole chunk": ("chunked", "_chunk", "Kbar = ratio[:, L - 1] * k", "Kbar = gamma[:, L - 1] * k"),
    # the backward (reverse of the step rule)
    "du -> dk term dropped": ("backward", "_step_grads",
                              "dk = dk + erase[..., None] * du\n        derase = np.sum(k * du, axis=-1) + np.sum(v * dm",
                              "derase = np.sum(k * du, axis=-1) + np.sum(v * dm"),
    "dalpha against the new state": ("backward", "_step_grads", "dalpha = np.sum(dX * S_prev, axis=-1)",
                                     "dalpha = np.sum(dX * S_t, axis=-1)"),
    "dq from the old state": ("backward", "_step_grads", 'dq = np.einsum("...ij,...j->...i", S_t, do)',
                              'dq = np.einsum("...ij,...j->...i", S_prev, do)'),
    "readout gradient not added": ("backward", "_step_grads", "G = G + q[..., :, None] * do[..., None, :]", "G = G"),
    "GDN-2 dk without the erase gate": ("backward", "_step_grads", "dk = dk + erase * du", "dk = dk + du"),
    "RDA write-gate gradient dropped": ("backward", "_step_grads", "dwrite = np.sum(v * dm, axis=-1)",
                                        "dwrite = 0.0 * np.sum(v * dm, axis=-1)"),
    # stored states
    "pool slot written for a sequence outside the pool": ("states", "pooled_prefill", "        if ok:\n            new[i] = S_T[n]",
                                                          "        if ok or i == -1:\n            new[i] = S_T[n]"),
    "snapshot one token early": ("states", "snapshots", "if (t - t0 + 1) % every == 0:", "if (t - t0) % every == 0:"),
    # two transitions per token (DeltaProduct page)
    "decay applied in both transitions": ("product", "product_step",
                                          'return step(S1, q, k[..., 1, :], v[..., 1, :], ones, beta[..., 1], None, "kda")',
                                          'return step(S1, q, k[..., 1, :], v[..., 1, :], alpha, beta[..., 1], None, "kda")'),
    "transitions in reverse order": ("product", "product_step",
                                     'S1, _ = step(S, q, k[..., 0, :], v[..., 0, :], alpha, beta[..., 0], None, "kda")',
                                     'S1, _ = step(S, q, k[..., 1, :], v[..., 1, :], alpha, beta[..., 1], None, "kda")'),
    # fused input preparation
    "tanh argument rescaled": ("prep", "alpha_from", "return np.tanh(z)", "return np.tanh(1.0001 * z)"),
    "softsign in place of tanh": ("prep", "alpha_from", "return np.tanh(z)", "return z / (1.0 + np.abs(z))"),
    "softplus decay rescaled": ("prep", "alpha_from", "return np.exp(-scale * softplus(z))",
                                "return np.exp(-1.01 * scale * softplus(z))"),
    "sigmoid argument rescaled": ("prep", "gate_from", "return scale * sigmoid(z)", "return scale * sigmoid(1.01 * z)"),
    "L2 norm with an epsilon": ("prep", "l2_normalize", "n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
                                "n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)"),
    # the error metric (max |err| / RMS)
    "error scaled by the mean magnitude": ("recurrence", "rel_err", "rms = float(np.sqrt(np.mean(ref * ref)))",
                                           "rms = float(np.mean(np.abs(ref)))"),
}


def plant(name):
    """Replace the oracle function named by MUTANTS[name] with its planted variant."""
    modname, fn, old, new = MUTANTS[name]
    mod = importlib.import_module("oracle." + modname)
    orig = getattr(mod, fn)
    src = textwrap.dedent(inspect.getsource(orig))
    if src.count(old) != 1:
        raise RuntimeError(f"mutant {name!r}: the statement is not in oracle.{modname}.{fn} exactly once")
    ns = {}
    exec(compile(src.replace(old, new), f"<planted: {name}>", "exec"), mod.__dict__, ns)
    planted = ns[fn]
    for m in list(sys.modules.values()):
        if getattr(m, "__name__", "").split(".")[0] == "oracle":
            for attr, val in list(vars(m).items()):
                if val is orig:
                    setattr(m, attr, planted)


def pytest_configure(config):
    name = os.environ.get("DR_ORACLE_MUTANT")
    if name:
        plant(name)
