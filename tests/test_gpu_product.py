"""GPU parity of the two-transitions-per-token variant ("product2": KDA's rule twice per
token, the decay once) against the fp64 oracle ``oracle.product``: prefill (fixed length,
ragged, packed, snapshots, state pools, fused input preparation, the full KDA prefill
shape on sampled pairs), decode (every head size, pools, fused preparation) and the
gradients (dr_chunk_bwd) against ``oracle.product.product_grads``.
Tolerance max |err| / RMS(ref): 1e-4 for fp32 inputs, 1e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
from oracle import prep, product, rel_err
import synth
from gpu_util import TOL, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy().astype(np.float64)


def _dev(wl, alpha_dtype=None):
    return dict(q=to_dev(wl.q, wl.in_dtype), k=to_dev(wl.k, wl.in_dtype), v=to_dev(wl.v, wl.in_dtype),
                alpha=to_dev(wl.alpha, alpha_dtype), erase=to_dev(wl.erase), write=None, variant="product2",
                S0=to_dev(wl.S0), cu_seqlens=None if wl.cu_seqlens is None else to_dev(wl.cu_seqlens))


def _check(tag, pairs, tol):
    errs = [rel_err(a, b) for a, b in pairs]
    print(f"[product2 {tag}] err " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    for e in errs:
        assert e <= tol, (tag, errs)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("recipe", ["kda", "ckda"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
def test_prefill(recipe, dk, dv, in_dtype):
    wl = synth.make_product(recipe, 2, 150, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("p2", recipe, dk, dv, in_dtype))
    o, S_T = drl.chunk_fwd(**_dev(wl))
    torch.cuda.synchronize()
    o_ref, S_ref = product.product_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, S0=wl.S0)
    _check(f"{recipe} d{dk}x{dv} {in_dtype}", [(_np(o), o_ref), (_np(S_T), S_ref)], TOL[in_dtype])


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 97])
def test_ragged_lengths(T):
    wl = synth.make_product("ckda", 1, T, 2, 64, 64, in_dtype="f32", seed=T)
    o, S_T = drl.chunk_fwd(**_dev(wl))
    torch.cuda.synchronize()
    o_ref, S_ref = product.product_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, S0=wl.S0)
    _check(f"T={T}", [(_np(o), o_ref), (_np(S_T), S_ref)], TOL["f32"])


def test_packed_sequences():
    lens = [70, 0, 1, 32, 129, 33]
    wl = synth.make_product("kda", 1, 0, 3, 128, 64, in_dtype="bf16", seed=seed_of("p2 packed"), lengths=lens)
    o, S_T = drl.chunk_fwd(**_dev(wl))
    torch.cuda.synchronize()
    o_ref, S_ref = product.product_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, S0=wl.S0,
                                              cu_seqlens=wl.cu_seqlens)
    _check("packed", [(_np(o), o_ref), (_np(S_T), S_ref)], TOL["bf16"])
    np.testing.assert_array_equal(_np(S_T)[1], wl.S0[1].astype(np.float64))  # empty sequence


def test_snapshots_every_32_tokens():
    lens = [100, 32, 0, 65]
    wl = synth.make_product("ckda", 1, 0, 2, 64, 64, in_dtype="f32", seed=seed_of("p2 snap"), lengths=lens)
    o, S_T, snaps = drl.chunk_fwd(**_dev(wl), snapshot_every=32)
    torch.cuda.synchronize()
    snaps = _np(snaps)
    assert snaps.shape[0] == drl.snapshot_count(lens, 32)
    row, cu = 0, wl.cu_seqlens
    for n, L in enumerate(lens):
        for j in range(L // 32):
            t1 = int(cu[n]) + 32 * (j + 1)
            sl = (slice(None), slice(int(cu[n]), t1))
            _, S_p = product.product_recurrence(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], wl.erase[sl],
                                                S0=wl.S0[n:n + 1])
            _check(f"snapshot n={n} j={j}", [(snaps[row], S_p[0])], TOL["f32"])
            row += 1
    assert row == snaps.shape[0]


def test_state_pool_prefill():
    wl = synth.make_product("kda", 3, 90, 2, 32, 32, in_dtype="f32", seed=seed_of("p2 pool"))
    rng = np.random.default_rng(7)
    pool = rng.standard_normal((5, 2, 32, 32)).astype(np.float32)
    idx = np.array([4, 0, 2], np.int32)
    a = _dev(wl)
    a["S0"] = to_dev(pool)
    o, S_T = drl.chunk_fwd(**a, state_idx=to_dev(idx))
    torch.cuda.synchronize()
    o_ref, S_ref = product.product_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, S0=pool[idx])
    after = pool.astype(np.float64).copy()
    after[idx] = S_ref
    _check("pool", [(_np(o), o_ref), (_np(S_T), after)], TOL["f32"])


@pytest.mark.parametrize("recipe", ["kda", "ckda"])
def test_fused_preparation(recipe):
    wl = synth.make_product(recipe, 2, 130, 2, 64, 64, in_dtype="bf16", seed=seed_of("p2 prep", recipe),
                            preact=True, alpha_dtype="bf16")
    kw = {k: v for k, v in wl.meta["prep"].items() if k != "alpha_dtype"}
    o, S_T = drl.chunk_fwd(**_dev(wl, "bf16"), prep=kw)
    torch.cuda.synchronize()
    q, k, alpha, beta, _ = prep.prepare(wl.q, wl.k, wl.alpha, wl.erase, None, **kw)
    o_ref, S_ref = product.product_recurrence(q, k, wl.v, alpha, beta, S0=wl.S0)
    _check(f"prep {recipe}", [(_np(o), o_ref), (_np(S_T), S_ref)], TOL["bf16"])


def test_full_size_sampled_pairs():
    # the KDA prefill shape (B=4, T=4096, H=16, d=128) with two transitions per token
    wl = synth.preset("product2_prefill")
    o, S_T = drl.chunk_fwd(**_dev(wl))
    torch.cuda.synchronize()
    o, S_T = _np(o), _np(S_T)
    for (n, h) in [(0, 3), (3, 15)]:
        sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        o_ref, S_ref = product.product_recurrence(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], wl.erase[sl],
                                                  S0=wl.S0[n:n + 1, h:h + 1])
        _check(f"full n={n} h={h}", [(o[n, :, h], o_ref[0, :, 0]), (S_T[n, h], S_ref[0, 0])], TOL["bf16"])


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (64, 64), (128, 32), (128, 128)])
def test_decode(dk, dv, in_dtype):
    wd = synth.make_product_decode("ckda", 6, 3, dk, dv, steps=3, in_dtype=in_dtype, seed=seed_of("p2 dec", dk, dv))
    S = to_dev(wd.S0)
    S_ref = wd.S0.astype(np.float64)
    for t in range(3):
        o = drl.decode_step(to_dev(wd.q[t], in_dtype), to_dev(wd.k[t], in_dtype), to_dev(wd.v[t], in_dtype),
                            to_dev(wd.alpha[t]), to_dev(wd.erase[t]), None, "product2", S)
        torch.cuda.synchronize()
        S_ref, o_ref = product.product_decode_step(S_ref, wd.q[t], wd.k[t], wd.v[t], wd.alpha[t], wd.erase[t])
        _check(f"decode d{dk}x{dv} {in_dtype} step {t}", [(_np(o), o_ref), (_np(S), S_ref)], 1e-4)


def test_decode_state_pool_and_preparation():
    N, H, d = 4, 2, 128
    wd = synth.make_product_decode("kda", N, H, d, d, steps=2, in_dtype="bf16", seed=seed_of("p2 dec pool"),
                                   preact=True, alpha_dtype="bf16")
    kw = {k: v for k, v in wd.meta["prep"].items() if k != "alpha_dtype"}
    rng = np.random.default_rng(3)
    pool = rng.standard_normal((7, H, d, d)).astype(np.float32)
    idx = np.array([6, 1, -1, 3], np.int32)    # -1: no state, output zero
    S = to_dev(pool)
    ref = pool.astype(np.float64).copy()
    for t in range(2):
        o = drl.decode_step(to_dev(wd.q[t], "bf16"), to_dev(wd.k[t], "bf16"), to_dev(wd.v[t], "bf16"),
                            to_dev(wd.alpha[t], "bf16"), to_dev(wd.erase[t]), None, "product2", S,
                            state_idx=to_dev(idx), prep=kw)
        torch.cuda.synchronize()
        q, k, alpha, beta, _ = prep.prepare(wd.q[t], wd.k[t], wd.alpha[t], wd.erase[t], None, **kw)
        live = idx >= 0
        S_new, o_ref = product.product_decode_step(ref[idx[live]], q[live], k[live], wd.v[t][live], alpha[live],
                                                   beta[live])
        ref[idx[live]] = S_new
        o_np = _np(o)
        _check(f"decode pool step {t}", [(o_np[live], o_ref), (_np(S), ref)], 1e-4)
        assert np.all(o_np[~live] == 0.0)


def _grads(wl, rng):
    a = _dev(wl)
    dO = rng.standard_normal(wl.q.shape[:3] + (wl.v.shape[-1],)).astype(np.float32)
    N = wl.num_seqs
    dS = rng.standard_normal((N,) + wl.S0.shape[1:]).astype(np.float32)
    g = drl.chunk_bwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], None, "product2", a["S0"], a["cu_seqlens"],
                      dO=to_dev(dO), dS_T=to_dev(dS))
    torch.cuda.synchronize()
    g = {k: (None if v is None else _np(v)) for k, v in g.items()}
    return g, dO, dS


NAMES = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dalpha", "dalpha"), ("derase", "dbeta"), ("dS0", "dS0"))


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("recipe", ["kda", "ckda"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128)])
def test_backward(recipe, dk, dv, in_dtype):
    wl = synth.make_product(recipe, 2, 75, 2, dk, dv, in_dtype=in_dtype, seed=seed_of("p2 bwd", recipe, dk, dv, in_dtype))
    g, dO, dS = _grads(wl, np.random.default_rng(seed_of("p2 bwd do", dk, dv)))
    ref = product.product_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, dO, dS_T=dS, S0=wl.S0)
    assert g["dwrite"] is None
    _check(f"backward {recipe} d{dk}x{dv} {in_dtype}", [(g[a], ref[b]) for a, b in NAMES], TOL[in_dtype])


def test_backward_packed():
    lens = [40, 0, 1, 33, 70]
    wl = synth.make_product("ckda", 1, 0, 2, 64, 64, in_dtype="f32", seed=seed_of("p2 bwd packed"), lengths=lens)
    g, dO, dS = _grads(wl, np.random.default_rng(4))
    ref = product.product_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, dO, dS_T=dS, S0=wl.S0,
                                cu_seqlens=wl.cu_seqlens)
    _check("backward packed", [(g[a], ref[b]) for a, b in NAMES], TOL["f32"])
    np.testing.assert_array_equal(g["dS0"][1], dS[1].astype(np.float64))  # empty sequence


def test_backward_full_size_sampled_pair():
    # the KDA prefill shape with two transitions per token; the oracle runs one (sequence, head)
    wl = synth.preset("product2_prefill")
    g, dO, dS = _grads(wl, np.random.default_rng(1006))
    n, h = 2, 7
    sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
    ref = product.product_grads(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], wl.erase[sl], dO[sl],
                                dS_T=dS[n:n + 1, h:h + 1], S0=wl.S0[n:n + 1, h:h + 1])
    pairs = [(g[a][sl], ref[b]) for a, b in NAMES if a != "dS0"] + [(g["dS0"][n, h], ref["dS0"][0, 0])]
    _check("backward full size", pairs, TOL["bf16"])


def test_backward_given_checkpoints():
    # the two-transition variant's checkpoints are the forward's snapshots every 32 tokens
    wl = synth.make_product("ckda", 2, 100, 2, 64, 64, in_dtype="bf16", seed=seed_of("p2 ckpt"))
    a = _dev(wl)
    _, _, snaps = drl.chunk_fwd(**a, snapshot_every=32)
    rng = np.random.default_rng(3)
    dO = to_dev(rng.standard_normal(wl.q.shape[:3] + (wl.v.shape[-1],)).astype(np.float32))
    g0 = drl.chunk_bwd(**a, dO=dO)
    g1 = drl.chunk_bwd(**a, dO=dO, checkpoints=snaps)
    torch.cuda.synchronize()
    for name, t in g0.items():
        assert (t is None and g1[name] is None) or torch.equal(t, g1[name]), name
