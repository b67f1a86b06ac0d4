"""GPU: the prefill of fixed-length batches runs in windows of chunk positions (the preparation and
the state pass over a few chunks of every sequence at a time, the state carried from one window to
the next). Splitting into windows changes no arithmetic: the results equal the one-window run bit for
bit, for every option of the prefill. DR_WINDOW_BYTES forces small windows."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
import synth
from gpu_util import TOL, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _run(monkeypatch, window_bytes, fn):
    if window_bytes is None:
        monkeypatch.delenv("DR_WINDOW_BYTES", raising=False)
    else:
        monkeypatch.setenv("DR_WINDOW_BYTES", str(window_bytes))
    out = fn()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("variant,dk,dv,in_dtype", [("kda", 128, 128, "bf16"), ("gdn2", 64, 32, "bf16"),
                                                    ("ckda", 32, 64, "f32"), ("rda", 16, 128, "bf16")])
@pytest.mark.parametrize("window_bytes", [1, 200_000])
def test_windows_equal_one_window(monkeypatch, variant, dk, dv, in_dtype, window_bytes):
    # T = 300: five chunks (the last partial); window_bytes 1 gives windows of one chunk
    wl = synth.make_prefill(variant, 3, 300, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("win", variant, dk, dv))
    a = prefill_inputs(wl)
    o1, s1 = _run(monkeypatch, None, lambda: drl.chunk_fwd(**a))
    o2, s2 = _run(monkeypatch, window_bytes, lambda: drl.chunk_fwd(**a))
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, S0=wl.S0)
    eo, es = oracle.rel_err(o2.cpu().numpy(), o_ref), oracle.rel_err(s2.cpu().numpy(), s_ref)
    assert eo <= TOL[in_dtype] and es <= TOL[in_dtype], (eo, es)


def test_windows_with_every_option(monkeypatch):
    """Snapshots, slot pools with an in-place state and an out-of-pool slot, the states-only call,
    fused input preparation and two transitions per token, each split into one-chunk windows."""
    wl = synth.make_prefill("kda", 3, 260, 2, 64, 64, in_dtype="bf16", seed=seed_of("win opts"))
    a = prefill_inputs(wl)
    f = lambda: drl.chunk_fwd(**a, snapshot_every=64)  # noqa: E731
    r1 = _run(monkeypatch, None, f)
    r2 = _run(monkeypatch, 1, f)
    assert all(torch.equal(x, y) for x, y in zip(r1, r2))
    f = lambda: drl.chunk_fwd(**a, output=False)  # noqa: E731
    assert torch.equal(_run(monkeypatch, None, f)[1], _run(monkeypatch, 1, f)[1])
    # slot pool: sequence n uses row idx[n] of a pool updated in place; row -1 is outside the pool
    pool0 = torch.randn((5, 2, 64, 64), device=a["q"].device)
    idx = torch.tensor([3, -1, 0], dtype=torch.int32, device=a["q"].device)

    def pooled():
        pool = pool0.clone()
        o, _ = drl.chunk_fwd(**dict(a, S0=pool), state_idx=idx)
        return o, pool
    p1, p2 = _run(monkeypatch, None, pooled), _run(monkeypatch, 1, pooled)
    assert torch.equal(p1[0], p2[0]) and torch.equal(p1[1], p2[1])
    # fused preparation
    wp = synth.make_prefill("ckda", 2, 200, 2, 64, 64, in_dtype="bf16", seed=seed_of("win prep"), preact=True,
                            alpha_dtype="bf16")
    ap = prefill_inputs(wp)
    ap["alpha"] = to_dev(wp.alpha, "bf16")
    kw = {k: v for k, v in wp.meta["prep"].items() if k != "alpha_dtype"}
    f = lambda: drl.chunk_fwd(**ap, prep=kw)  # noqa: E731
    r1, r2 = _run(monkeypatch, None, f), _run(monkeypatch, 1, f)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    # two transitions per token
    w2 = synth.make_product("kda", 2, 100, 2, 64, 64, in_dtype="bf16", seed=seed_of("win p2"))
    a2 = prefill_inputs(w2)
    f = lambda: drl.chunk_fwd(**a2)  # noqa: E731
    r1, r2 = _run(monkeypatch, None, f), _run(monkeypatch, 1, f)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_backward_with_windowed_checkpointing_forward(monkeypatch):
    wl = synth.make_prefill("rda", 2, 200, 2, 64, 64, in_dtype="bf16", seed=seed_of("win bwd"))
    a = prefill_inputs(wl)
    dO = torch.randn(a["q"].shape[:3] + (64,), device=a["q"].device)
    f = lambda: drl.chunk_bwd(**a, dO=dO)  # noqa: E731
    g1, g2 = _run(monkeypatch, None, f), _run(monkeypatch, 1, f)
    for key in g1:
        if g1[key] is not None:
            assert torch.equal(g1[key], g2[key]), key


def test_million_token_sequence_in_a_fixed_workspace(monkeypatch):
    """One sequence of 2^20 tokens (2 heads, d = 64, bf16): the prefill runs in windows within a
    workspace of about 150 MB whatever the length. Its first 16384 outputs match the oracle run
    on those tokens alone (a prefix does not depend on what follows), and the whole run equals,
    bit for bit, the same tokens in two calls split at a chunk boundary, the second resuming from
    the first's final state."""
    monkeypatch.delenv("DR_WINDOW_BYTES", raising=False)
    T, H, d = 1 << 20, 2, 64
    plan = drl.chunk_fwd_plan_ex(1, T, H, d, d)
    print(f"[windows 1M] plan {plan}", flush=True)
    assert plan["windows"] > 10 and plan["workspace"] < 160 * 2 ** 20, plan
    wl = synth.make_prefill("kda", 1, T, H, d, d, in_dtype="bf16", seed=seed_of("million"))
    a = prefill_inputs(wl)
    o, S = drl.chunk_fwd(**a)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    n = 16384
    oo, _ = oracle.step_recurrence(wl.q[:, :n], wl.k[:, :n], wl.v[:, :n], wl.alpha[:, :n], wl.erase[:, :n], None,
                                   "kda", S0=wl.S0)
    e = oracle.rel_err(o[:, :n].cpu().numpy(), oo)
    print(f"[windows 1M] first {n} tokens against the oracle: err o={e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    h = T // 2
    sl = lambda x, lo, hi: None if x is None else x[:, lo:hi].contiguous()  # noqa: E731
    first = {key: (sl(val, 0, h) if key in ("q", "k", "v", "alpha", "erase", "write") else val)
             for key, val in a.items()}
    o1, S1 = drl.chunk_fwd(**first)
    second = {key: (sl(val, h, T) if key in ("q", "k", "v", "alpha", "erase", "write") else val)
              for key, val in a.items()}
    second["S0"] = S1
    o2, S2 = drl.chunk_fwd(**second)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=1), o) and torch.equal(S2, S)
    print("[windows 1M] split run identical bit for bit", flush=True)
