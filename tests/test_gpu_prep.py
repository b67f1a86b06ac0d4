"""GPU parity of the fused input preparation (dr_chunk_fwd_ex / dr_decode_step_ex with the
``l2norm_qk`` / ``alpha_act`` / ``gate_act`` options): the kernels take raw q, k and gate
pre-activations, the oracle prepares them with ``oracle.prep`` in float64 and runs the
recurrence. Tolerance as for the plain calls: max |err| / RMS(ref) <= 1e-4 (fp32 inputs),
1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
from oracle import prep
import synth
from gpu_util import TOL, decode_inputs, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy().astype(np.float64)


def _kw(wl):
    return {k: v for k, v in wl.meta["prep"].items() if k != "alpha_dtype"}


def _inputs(wl):
    a = prefill_inputs(wl)
    a["alpha"] = to_dev(wl.alpha, wl.meta["prep"]["alpha_dtype"])
    return a


def _oracle(wl, sl=None):
    g = (lambda x: None if x is None else x[sl]) if sl is not None else (lambda x: x)
    q, k, alpha, erase, write = prep.prepare(g(wl.q), g(wl.k), g(wl.alpha), g(wl.erase), g(wl.write), **_kw(wl))
    return q, k, alpha, erase, write


@pytest.mark.parametrize("alpha_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
def test_prepared_prefill(variant, in_dtype, alpha_dtype):
    wl = synth.make_prefill(variant, 2, 150, 2, 64, 32, in_dtype=in_dtype, seed=seed_of("prep", variant, in_dtype),
                            preact=True, alpha_dtype=alpha_dtype)
    o, S_T = drl.chunk_fwd(**_inputs(wl), prep=_kw(wl))
    torch.cuda.synchronize()
    q, k, alpha, erase, write = _oracle(wl)
    o_ref, S_ref = oracle.step_recurrence(q, k, wl.v, alpha, erase, write, wl.variant, S0=wl.S0)
    eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S_T), S_ref)
    print(f"[prep prefill {variant} {in_dtype} alpha {alpha_dtype}] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= TOL[in_dtype] and es <= TOL[in_dtype]


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_prepared_prefill_narrow_keys(variant, in_dtype):
    """d_k = 16, below the 32-deep MFMA slice: lanes past d_k load channel 0 and must drop it from
    the norms and the gates (a ragged tail of 150 tokens besides)."""
    wl = synth.make_prefill(variant, 2, 150, 2, 16, 16, in_dtype=in_dtype, seed=seed_of("prep16", variant, in_dtype),
                            preact=True, alpha_dtype="f32")
    o, S_T = drl.chunk_fwd(**_inputs(wl), prep=_kw(wl))
    torch.cuda.synchronize()
    q, k, alpha, erase, write = _oracle(wl)
    o_ref, S_ref = oracle.step_recurrence(q, k, wl.v, alpha, erase, write, wl.variant, S0=wl.S0)
    eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S_T), S_ref)
    print(f"[prep prefill d_k=16 {variant} {in_dtype}] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= TOL[in_dtype] and es <= TOL[in_dtype]


def test_prepared_prefill_d128_packed():
    lens = [130, 0, 64, 300, 1]
    wl = synth.make_prefill("gdn2", 1, 0, 3, 128, 128, in_dtype="bf16", seed=seed_of("prep", "packed"),
                            lengths=lens, preact=True, alpha_dtype="bf16")
    o, S_T = drl.chunk_fwd(**_inputs(wl), prep=_kw(wl))
    torch.cuda.synchronize()
    q, k, alpha, erase, write = _oracle(wl)
    o_ref, S_ref = oracle.step_recurrence(q, k, wl.v, alpha, erase, write, wl.variant, S0=wl.S0,
                                          cu_seqlens=wl.cu_seqlens)
    eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S_T), S_ref)
    print(f"[prep packed gdn2] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_infinite_preactivations_give_exact_gates():
    # Complex KDA: tanh(+-inf) = +-1 (orthogonal decay), 2 sigmoid(+inf) = 2 (a reflection),
    # so with every gate at its limit the state's Frobenius norm is preserved exactly in fp64
    # and to rounding on the GPU
    B, T, H, d = 1, 128, 2, 32
    rng = np.random.default_rng(3)
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    k = rng.standard_normal((B, T, H, d)).astype(np.float32)
    v = np.zeros((B, T, H, d), np.float32)
    za = np.where(rng.random((B, T, H, d)) < 0.5, -np.inf, np.inf).astype(np.float32)
    zb = np.where(rng.random((B, T, H)) < 0.5, -np.inf, np.inf).astype(np.float32)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    kw = dict(l2norm_qk=True, alpha_act="tanh", alpha_scale=1.0, gate_act="sigmoid", gate_scale=2.0)
    _, S_T = drl.chunk_fwd(to_dev(q), to_dev(k), to_dev(v), to_dev(za), to_dev(zb), None, "ckda", to_dev(S0), prep=kw)
    torch.cuda.synchronize()
    n0 = np.linalg.norm(S0.astype(np.float64), axis=(-2, -1))
    n1 = np.linalg.norm(_np(S_T), axis=(-2, -1))
    print(f"[prep limits] |S0|={n0} |S_T|={n1}", flush=True)
    np.testing.assert_allclose(n1, n0, rtol=1e-4)
    qp, kp, ap, bp, _ = prep.prepare(q, k, za, zb, None, **kw)
    assert set(np.unique(ap)) <= {-1.0, 1.0} and set(np.unique(bp)) <= {0.0, 2.0}
    _, S_ref = oracle.step_recurrence(qp, kp, v, ap, bp, None, "ckda", S0=S0)
    assert oracle.rel_err(_np(S_T), S_ref) <= 1e-4


def test_prepared_kda_prefill_workload_sampled():
    # the measured shape (B=4, T=4096, H=16, d=128) with raw q/k and bf16 decay pre-activations
    wl = synth.make_prefill("kda", 4, 4096, 16, 128, 128, in_dtype="bf16", seed=1002, preact=True,
                            alpha_dtype="bf16")
    o, S_T = drl.chunk_fwd(**_inputs(wl), prep=_kw(wl))
    torch.cuda.synchronize()
    o, S_T = _np(o), _np(S_T)
    for (n, h) in [(0, 0), (3, 15), (1, 9)]:
        sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        q, k, alpha, erase, _ = _oracle(wl, sl)
        o_ref, S_ref = oracle.step_recurrence(q, k, wl.v[sl], alpha, erase, None, "kda", S0=wl.S0[n:n + 1, h:h + 1])
        eo = oracle.rel_err(o[n, :, h], o_ref[0, :, 0])
        es = oracle.rel_err(S_T[n, h], S_ref[0, 0])
        print(f"[prep kda_prefill n={n} h={h}] err o={eo:.3e} S_T={es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("variant", ["kda", "rda", "gdn2", "ckda"])
def test_prepared_decode(variant):
    N, H, d = 8, 4, 128
    wd = synth.make_decode(variant, N, H, d, d, steps=3, in_dtype="bf16", seed=seed_of("prep dec", variant),
                           preact=True, alpha_dtype="bf16")
    kw = {k: v for k, v in wd.meta["prep"].items() if k != "alpha_dtype"}
    S = to_dev(wd.S0)
    S_ref = wd.S0.astype(np.float64)
    for t in range(3):
        a = decode_inputs(wd, t)
        a["alpha"] = to_dev(wd.alpha[t], "bf16")
        o = drl.decode_step(**a, S=S, prep=kw)
        torch.cuda.synchronize()
        q, k, alpha, erase, write = prep.prepare(wd.q[t], wd.k[t], wd.alpha[t], wd.erase[t],
                                                 None if wd.write is None else wd.write[t], **kw)
        S_ref, o_ref = oracle.decode_step(S_ref, q, k, wd.v[t], alpha, erase, write, variant)
        eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S), S_ref)
        print(f"[prep decode {variant} step {t}] err o={eo:.3e} S={es:.3e}", flush=True)
        assert eo <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("act,scale", [("exp_neg_softplus", 0.01), ("exp_neg_softplus", 0.1),
                                       ("exp_neg_softplus", 0.0), ("tanh", 1.0)])
def test_extreme_and_small_preactivations(act, scale):
    """Decay pre-activations spread from -1e3 to 1e3 (exp(-c softplus(z)) must follow exp(-c z) for
    large z instead of collapsing to 0, and give exactly 1 for c = 0) and crowded near 0 (tanh's
    small-argument range), in the prefill (fp32 and bf16 alpha) and the decode step."""
    B, T, H, d = 1, 150, 2, 64
    rng = np.random.default_rng(seed_of("extreme", act, scale))
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    k = rng.standard_normal((B, T, H, d)).astype(np.float32)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    mag = np.where(rng.random((B, T, H, d)) < 0.5, 10.0 ** rng.uniform(-4, 0, (B, T, H, d)),
                   10.0 ** rng.uniform(0, 3, (B, T, H, d)))
    za = (np.sign(rng.standard_normal((B, T, H, d))) * mag).astype(np.float32)
    zb = rng.standard_normal((B, T, H)).astype(np.float32)
    S0 = (rng.standard_normal((B, H, d, d)) / np.sqrt(d)).astype(np.float32)
    kw = dict(l2norm_qk=True, alpha_act=act, alpha_scale=scale, gate_act="sigmoid", gate_scale=1.0)
    variant = "ckda" if act == "tanh" else "kda"
    for adt in ("f32", "bf16"):
        za_d = to_dev(za, adt)
        z_used = za_d.float().cpu().numpy()   # the values the kernel sees (bf16-rounded for bf16 alpha)
        o, S_T = drl.chunk_fwd(to_dev(q), to_dev(k), to_dev(v), za_d, to_dev(zb), None, variant, to_dev(S0), prep=kw)
        torch.cuda.synchronize()
        qp, kp, ap, bp, _ = prep.prepare(q, k, z_used, zb, None, **kw)
        assert np.all(np.isfinite(ap))
        o_ref, S_ref = oracle.step_recurrence(qp, kp, v, ap, bp, None, variant, S0=S0)
        eo, es = oracle.rel_err(_np(o), o_ref), oracle.rel_err(_np(S_T), S_ref)
        print(f"[prep extreme {act} c={scale} alpha {adt}] err o={eo:.3e} S_T={es:.3e}", flush=True)
        assert eo <= TOL["f32"] and es <= TOL["f32"], (eo, es)
    # decode: one step per token of the first four
    S = to_dev(S0[0])[None].contiguous()
    S_ref = S0[0][None].astype(np.float64)
    for t in range(4):
        sl = lambda x: np.ascontiguousarray(x[:, t])  # noqa: E731
        od = drl.decode_step(to_dev(sl(q)), to_dev(sl(k)), to_dev(sl(v)), to_dev(sl(za)), to_dev(sl(zb)), None,
                             variant, S, prep=kw)
        qp, kp, ap, bp, _ = prep.prepare(sl(q), sl(k), sl(za), sl(zb), None, **kw)
        S_ref, od_ref = oracle.decode_step(S_ref, qp, kp, sl(v), ap, bp, None, variant)
    torch.cuda.synchronize()
    eo, es = oracle.rel_err(_np(od), od_ref), oracle.rel_err(_np(S), S_ref)
    print(f"[prep extreme decode {act} c={scale}] err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= TOL["f32"] and es <= TOL["f32"], (eo, es)
