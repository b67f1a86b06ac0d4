"""GPU: q, k and v given through strides (a dr_dims_v2), e.g. as views of one fused projection.
The kernels read them in place (no copy is made): the results of the prefill, the decode step and
the backward must equal the same call on contiguous copies bit for bit (the same values reach the
same instructions), and match the oracle."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
import synth
from gpu_util import TOL, decode_inputs, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _fused(parts, dtype):
    """One [..., len(parts), ...] tensor holding the given tensors along a new axis 2 (the
    layout of a fused projection), and the views of it that stand for each of them."""
    big = torch.stack(parts, dim=2).contiguous()
    views = [big[:, :, i] for i in range(len(parts))]
    for v_, p_ in zip(views, parts):
        assert not v_.is_contiguous() and torch.equal(v_, p_)
    return big, views


def _call(a, q, k, v):
    B, T, H, dk = a["q"].shape
    dv = a["v"].shape[-1]
    N = B if a["cu_seqlens"] is None else a["cu_seqlens"].shape[0] - 1
    o = torch.full((B, T, H, dv), 7.0, dtype=torch.float32, device=q.device)
    S = torch.full((N, H, dk, dv), 7.0, dtype=torch.float32, device=q.device)
    drl.dr_chunk_fwd(q, k, v, a["alpha"], a["erase"], a["write"], a["variant"], a["S0"], a["cu_seqlens"], o, S)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("variant,dk,in_dtype", [("kda", 128, "bf16"), ("gdn2", 64, "bf16"), ("ckda", 32, "f32"),
                                                 ("rda", 128, "f32")])
def test_views_of_one_projection(variant, dk, in_dtype):
    # q, k, v of equal head size from one [B, T, 3, H, d] tensor: token stride 3 H d
    wl = synth.make_prefill(variant, 2, 200, 3, dk, dk, in_dtype=in_dtype, seed=seed_of("strided", variant, dk))
    a = prefill_inputs(wl)
    big, (q, k, v) = _fused([a["q"], a["k"], a["v"]], a["q"].dtype)
    o_ref, S_ref = _call(a, a["q"], a["k"], a["v"])
    o, S = _call(a, q, k, v)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    oo, so = oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, S0=wl.S0)
    eo, es = oracle.rel_err(o.cpu().numpy(), oo), oracle.rel_err(S.cpu().numpy(), so)
    print(f"[strided {variant} d={dk} {in_dtype}] err o={eo:.3e} S_T={es:.3e}", flush=True)
    assert eo <= TOL[in_dtype] and es <= TOL[in_dtype]


def test_slices_along_time_and_packed_views():
    # a batch stride that is not T times the token stride: the first 130 tokens of 160-token rows,
    # q, k, v from three different buffers
    wl = synth.make_prefill("kda", 3, 130, 2, 64, 32, in_dtype="bf16", seed=seed_of("strided slice"))
    a = prefill_inputs(wl)
    views = []
    for name in ("q", "k", "v"):
        x = a[name]
        pad = torch.randn((x.shape[0], 160) + x.shape[2:], device=x.device).to(x.dtype)
        pad[:, :130] = x
        views.append(pad[:, :130])
        assert views[-1].stride(0) == 160 * views[-1].stride(1)
    o_ref, S_ref = _call(a, a["q"], a["k"], a["v"])
    o, S = _call(a, *views)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    # packed sequences (one batch row, offsets) from a fused projection
    wl = synth.make_prefill("gdn2", 1, 0, 2, 64, 64, in_dtype="bf16", seed=seed_of("strided packed"),
                            lengths=[40, 0, 97, 1, 64])
    a = prefill_inputs(wl)
    big, (q, k, v) = _fused([a["q"], a["k"], a["v"]], a["q"].dtype)
    o_ref, S_ref = _call(a, a["q"], a["k"], a["v"])
    o, S = _call(a, q, k, v)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_two_transitions_per_token_views():
    # k and v [B, T, H, 2, d] as views of [B, T, 2, H, 2, d] tensors (their two steps stay d apart)
    wl = synth.make_product("kda", 2, 70, 2, 64, 64, in_dtype="bf16", seed=seed_of("strided product"))
    a = prefill_inputs(wl)
    kbig = torch.stack([a["k"], torch.zeros_like(a["k"])], dim=2).contiguous()
    vbig = torch.stack([torch.zeros_like(a["v"]), a["v"]], dim=2).contiguous()
    k, v = kbig[:, :, 0], vbig[:, :, 1]
    assert not k.is_contiguous() and torch.equal(k, a["k"])
    o_ref, S_ref = _call(a, a["q"], a["k"], a["v"])
    o, S = _call(a, a["q"], k, v)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("variant", ["kda", "gdn2", "product2"])
def test_decode_views(variant):
    if variant == "product2":
        wl = synth.make_product_decode("kda", 6, 3, 64, 64, steps=1, in_dtype="bf16", seed=seed_of("strided dec p2"))
    else:
        wl = synth.make_decode(variant, 6, 3, 128, 128, steps=1, in_dtype="bf16", seed=seed_of("strided dec", variant))
    a = decode_inputs(wl, 0)
    # q, k, v [N, H, ...] as views of an [N, 3, H, ...] projection (stride between sequences 3 H d)
    if variant == "product2":
        q = torch.stack([a["q"], a["q"]], dim=1).contiguous()[:, 1]
        k = torch.stack([a["k"], a["k"]], dim=1).contiguous()[:, 0]
        v = torch.stack([a["v"], a["v"]], dim=1).contiguous()[:, 1]
    else:
        big = torch.stack([a["q"], a["k"], a["v"]], dim=1).contiguous()
        q, k, v = big[:, 0], big[:, 1], big[:, 2]
    assert not q.is_contiguous()
    S1 = to_dev(wl.S0).clone()
    S2 = S1.clone()
    o1 = drl.decode_step(S=S1, **a)
    o2 = drl.decode_step(S=S2, **dict(a, q=q, k=k, v=v))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("case", ["kda", "gdn2_packed", "product2"])
def test_backward_on_views(case):
    # the backward reads q, k, v through their strides too: gradients equal those of the call on
    # contiguous copies bit for bit (the gradients themselves are dense)
    if case == "kda":
        wl = synth.make_prefill("kda", 2, 150, 2, 128, 128, in_dtype="bf16", seed=seed_of("strided bwd", case))
    elif case == "gdn2_packed":
        wl = synth.make_prefill("gdn2", 1, 0, 2, 64, 64, in_dtype="bf16", seed=seed_of("strided bwd", case),
                                lengths=[70, 0, 1, 129])
    else:
        wl = synth.make_product("kda", 2, 77, 2, 64, 64, in_dtype="bf16", seed=seed_of("strided bwd", case))
    a = prefill_inputs(wl)
    if case == "product2":  # k, v [B, T, H, 2, d] as views of [B, T, 2, H, 2, d] tensors
        k = torch.stack([a["k"], torch.zeros_like(a["k"])], dim=2).contiguous()[:, :, 0]
        v = torch.stack([torch.zeros_like(a["v"]), a["v"]], dim=2).contiguous()[:, :, 1]
        q = torch.stack([a["q"], a["q"]], dim=2).contiguous()[:, :, 1]
    else:
        big, (q, k, v) = _fused([a["q"], a["k"], a["v"]], a["q"].dtype)
    assert not (q.is_contiguous() or k.is_contiguous() or v.is_contiguous())
    gen = torch.Generator(device="cuda").manual_seed(seed_of("strided bwd do", case))
    dO = torch.randn(a["q"].shape[:3] + (a["v"].shape[-1],), device="cuda", generator=gen)
    N = wl.S0.shape[0]
    dS_T = torch.randn((N,) + tuple(wl.S0.shape[1:]), device="cuda", generator=gen)
    g_ref = drl.chunk_bwd(**a, dO=dO, dS_T=dS_T)
    g = drl.chunk_bwd(**dict(a, q=q, k=k, v=v), dO=dO, dS_T=dS_T)
    torch.cuda.synchronize()
    for name, ref in g_ref.items():
        assert (ref is None and g[name] is None) or torch.equal(g[name], ref), name
