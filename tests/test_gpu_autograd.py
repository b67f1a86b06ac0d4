"""GPU: the prefill as a torch autograd node (``delta_rule``). Gradients reached through
``backward()`` must equal those of a direct ``chunk_bwd`` call with the same dL/do and dL/dS_T bit
for bit (the same kernels run; the forward's checkpoints replace the backward's own recomputation,
which gives identical states), with and without checkpoints, for every variant, fixed and packed
sequences, strided inputs and losses on o alone; one case is also checked against the fp64
oracle's reverse recurrence."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import synth
from oracle import backward, rel_err
from gpu_util import TOL, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu

GRAD_OF = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("alpha", "dalpha"), ("erase", "derase"), ("write", "dwrite"),
           ("S0", "dS0"))


def _leaves(a):
    """The workload's float tensors as fresh leaves that require gradients."""
    x = dict(a)
    for name, _ in GRAD_OF:
        if x[name] is not None:
            x[name] = x[name].detach().clone().requires_grad_(True)
    return x


def _case(name):
    if name == "kda":
        return synth.make_prefill("kda", 2, 150, 2, 128, 128, in_dtype="bf16", seed=seed_of("autograd", name))
    if name == "gdn2_packed":
        return synth.make_prefill("gdn2", 1, 0, 2, 64, 64, in_dtype="bf16", seed=seed_of("autograd", name),
                                  lengths=[70, 0, 1, 129])
    if name == "rda_f32":
        return synth.make_prefill("rda", 2, 100, 2, 64, 32, in_dtype="f32", seed=seed_of("autograd", name))
    if name == "ckda":
        return synth.make_prefill("ckda", 1, 200, 3, 64, 64, in_dtype="bf16", seed=seed_of("autograd", name))
    return synth.make_product("kda", 2, 77, 2, 64, 64, in_dtype="bf16", seed=seed_of("autograd", name))


@pytest.mark.parametrize("checkpoint", [True, False])
@pytest.mark.parametrize("name", ["kda", "gdn2_packed", "rda_f32", "ckda", "product2"])
def test_autograd_matches_direct_backward(name, checkpoint):
    wl = _case(name)
    a = prefill_inputs(wl)
    x = _leaves(a)
    o, S_T = drl.delta_rule(x["q"], x["k"], x["v"], x["alpha"], x["erase"], x["write"], x["variant"], x["S0"],
                            x["cu_seqlens"], checkpoint=checkpoint)
    gen = torch.Generator(device="cuda").manual_seed(seed_of("autograd w", name))
    W = torch.randn(o.shape, device="cuda", generator=gen)
    V = torch.randn(S_T.shape, device="cuda", generator=gen)
    ((o * W).sum() + (S_T * V).sum()).backward()
    g = drl.chunk_bwd(**a, dO=W, dS_T=V)
    torch.cuda.synchronize()
    for name_in, name_g in GRAD_OF:
        if x[name_in] is None:
            assert g[name_g] is None, name_g
            continue
        got = x[name_in].grad
        assert got is not None and got.dtype == x[name_in].dtype, name_in
        assert torch.equal(got, g[name_g].to(got.dtype)), name_in


def test_loss_on_outputs_only_and_strided_views():
    wl = _case("kda")
    a = prefill_inputs(wl)
    # q, k, v as views of one fused [B, T, 3, H, d] projection: the forward reads them in place
    big = torch.stack([a["q"], a["k"], a["v"]], dim=2).detach().clone().requires_grad_(True)
    q, k, v = big[:, :, 0], big[:, :, 1], big[:, :, 2]
    x = _leaves(dict(a, q=None, k=None, v=None))
    o, S_T = drl.delta_rule(q, k, v, x["alpha"], x["erase"], None, "kda", x["S0"], None)
    gen = torch.Generator(device="cuda").manual_seed(seed_of("autograd o only"))
    W = torch.randn(o.shape, device="cuda", generator=gen)
    (o * W).sum().backward()
    g = drl.chunk_bwd(**a, dO=W)
    torch.cuda.synchronize()
    assert torch.equal(big.grad, torch.stack([g["dq"], g["dk"], g["dv"]], dim=2).to(big.dtype))
    assert torch.equal(x["alpha"].grad, g["dalpha"]) and torch.equal(x["erase"].grad, g["derase"])
    assert torch.equal(x["S0"].grad, g["dS0"])


def test_autograd_against_the_oracle():
    wl = synth.make_prefill("gdn2", 2, 90, 2, 32, 32, in_dtype="f32", seed=seed_of("autograd oracle"))
    x = _leaves(prefill_inputs(wl))
    o, S_T = drl.delta_rule(x["q"], x["k"], x["v"], x["alpha"], x["erase"], x["write"], "gdn2", x["S0"], None)
    rng = np.random.default_rng(seed_of("autograd oracle do"))
    dO = rng.standard_normal(o.shape).astype(np.float32)
    dS_T = rng.standard_normal(S_T.shape).astype(np.float32)
    ((o * to_dev(dO)).sum() + (S_T * to_dev(dS_T)).sum()).backward()
    ref = backward.step_recurrence_grads(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, "gdn2", dO, dS_T=dS_T,
                                         S0=wl.S0)
    for name_in, name_g in GRAD_OF:
        if x[name_in] is None:
            continue
        e = rel_err(x[name_in].grad.double().cpu().numpy(), ref[name_g])
        print(f"[autograd gdn2 f32] {name_g} err={e:.2e}", flush=True)
        assert e <= TOL["f32"], (name_g, e)
