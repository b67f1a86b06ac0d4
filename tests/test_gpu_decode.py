"""GPU parity of the decode step (dr_decode_step) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
import synth
from gpu_util import seed_of, TOL, decode_inputs, prefill_inputs, to_dev

pytestmark = pytest.mark.gpu


def _oracle_step(wl, S, t, sel=None):
    g = lambda x: None if x is None else (x[t] if sel is None else x[t][sel])  # noqa: E731
    return oracle.decode_step(S, g(wl.q), g(wl.k), g(wl.v), g(wl.alpha), g(wl.erase), g(wl.write),
                              wl.variant)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (64, 64), (128, 128), (128, 16)])
def test_small_steps(variant, dk, dv, in_dtype):
    wl = synth.make_decode(variant, 5, 3, dk, dv, steps=4, in_dtype=in_dtype,
                           seed=seed_of(variant, dk, dv))
    S = to_dev(wl.S0).clone()
    S_ref = wl.S0.astype(np.float64)
    tol = TOL[in_dtype]
    for t in range(4):
        o = drl.decode_step(S=S, **decode_inputs(wl, t))
        S_ref, o_ref = _oracle_step(wl, S_ref, t)
        torch.cuda.synchronize()
        eo = oracle.rel_err(o.cpu().numpy(), o_ref)
        es = oracle.rel_err(S.cpu().numpy(), S_ref)
        assert eo <= tol and es <= tol, (t, eo, es)
    print(f"[decode {variant} {dk}x{dv} {in_dtype}] err o={eo:.3e} S={es:.3e}", flush=True)


def test_decode_steps_match_prefill():
    """T decode steps and one prefill of the same T tokens give the same result."""
    wl = synth.make_prefill("gdn2", 2, 40, 3, 128, 128, in_dtype="bf16", seed=7)
    a = prefill_inputs(wl)
    o_p, S_p = drl.chunk_fwd(**a)
    S = a["S0"].clone()
    outs = []
    for t in range(40):
        sl = lambda x: None if x is None else x[:, t].contiguous()  # noqa: E731
        outs.append(drl.decode_step(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(a["alpha"]), sl(a["erase"]),
                                    sl(a["write"]), "gdn2", S))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    assert oracle.rel_err(o_d.cpu().numpy(), o_p.cpu().numpy()) < 1e-4
    assert oracle.rel_err(S.cpu().numpy(), S_p.cpu().numpy()) < 1e-4


def test_kda_is_rda_with_equal_gates_bitwise():
    wl = synth.make_decode("kda", 8, 4, 128, 128, steps=1, seed=8)
    a = decode_inputs(wl, 0)
    S1 = to_dev(wl.S0).clone()
    S2 = S1.clone()
    o1 = drl.decode_step(S=S1, **a)
    o2 = drl.decode_step(S=S2, **dict(a, variant="rda", write=a["erase"].clone()))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
def test_full_size_decode(variant):
    """512 sequences x 32 heads x 128 x 128 fp32 state (1 GiB) updated in place. Step 1 is
    checked on every head; after 10, 100 and 1000 consecutive steps (inputs cycled from a pool
    of 16 distinct token sets) 64 seeded heads are checked."""
    pool = 16
    wl = synth.preset(f"decode_{variant}", steps=pool)
    N, H = wl.S0.shape[:2]
    S = to_dev(wl.S0)
    toks = [decode_inputs(wl, t) for t in range(pool)]
    tol = TOL["bf16"]
    o = drl.decode_step(S=S, **toks[0])
    torch.cuda.synchronize()
    o_np, S_np = o.cpu().numpy(), S.cpu().numpy()
    err_o = err_s = 0.0
    num = np.zeros(2); den = np.zeros(2)
    for n0 in range(0, N, 64):       # all heads, in slices to bound host memory
        sl = slice(n0, n0 + 64)
        S_ref, o_ref = _oracle_step(wl, wl.S0[sl].astype(np.float64), 0, sel=sl)
        err_o = max(err_o, np.max(np.abs(o_np[sl] - o_ref)))
        err_s = max(err_s, np.max(np.abs(S_np[sl] - S_ref)))
        num += [np.sum(o_ref ** 2), np.sum(S_ref ** 2)]
        den += [o_ref.size, S_ref.size]
    eo, es = err_o / np.sqrt(num[0] / den[0]), err_s / np.sqrt(num[1] / den[1])
    print(f"[decode full {variant}] step 1 all heads: err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= tol and es <= tol
    rng = np.random.default_rng(5)
    idx = rng.choice(N * H, 64, replace=False)
    ns, hs = idx // H, idx % H
    S_ref = wl.S0[ns, hs].astype(np.float64)
    S_ref, _ = oracle.decode_step(S_ref, wl.q[0][ns, hs], wl.k[0][ns, hs], wl.v[0][ns, hs],
                                  wl.alpha[0][ns, hs], wl.erase[0][ns, hs],
                                  None if wl.write is None else wl.write[0][ns, hs], variant)
    for step in range(1, 1000):
        t = step % pool
        o = drl.decode_step(S=S, **toks[t])
        S_ref, o_ref = oracle.decode_step(S_ref, wl.q[t][ns, hs], wl.k[t][ns, hs], wl.v[t][ns, hs],
                                          wl.alpha[t][ns, hs], wl.erase[t][ns, hs],
                                          None if wl.write is None else wl.write[t][ns, hs], variant)
        if step + 1 in (10, 100, 1000):
            torch.cuda.synchronize()
            eo = oracle.rel_err(o.cpu().numpy()[ns, hs], o_ref)
            es = oracle.rel_err(S.cpu().numpy()[ns, hs], S_ref)
            print(f"[decode full {variant}] step {step + 1}, 64 heads: err o={eo:.3e} S={es:.3e}", flush=True)
            assert eo <= tol and es <= tol


def test_nan_stays_in_its_head():
    """NaN / Inf in one head's token leave every other head's output and state bit for bit as in
    a clean step (no two requests share a state: the course page "GDN, KDA và Mamba-2", section 3)."""
    for variant in ("kda", "gdn2"):
        wl = synth.make_decode(variant, 6, 4, 128, 128, steps=1, seed=seed_of("nan decode", variant))
        a = decode_inputs(wl, 0)
        S1 = to_dev(wl.S0).clone()
        S2 = S1.clone()
        o1 = drl.decode_step(S=S1, **a)
        b = {key: (x.clone() if torch.is_tensor(x) else x) for key, x in a.items()}
        b["q"][2, 1, 5] = float("nan")
        b["v"][2, 1, 0] = float("inf")
        b["alpha"][2, 1, 9] = float("nan")
        o2 = drl.decode_step(S=S2, **b)
        torch.cuda.synchronize()
        keep = torch.ones(o1.shape[:2], dtype=torch.bool, device=o1.device)
        keep[2, 1] = False
        assert not torch.isfinite(o2[2, 1]).all()
        assert torch.equal(o1[keep], o2[keep]) and torch.equal(S1[keep], S2[keep])
