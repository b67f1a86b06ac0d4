"""The decode step and the prefill captured in HIP graphs (torch.cuda.CUDAGraph on ROCm). The
decode step allocates nothing and never synchronises; the prefill takes its workspace
stream-ordered, which the capture records as memory nodes. Each replay is checked against the
same call run eagerly (same kernels, same inputs: bit-identical), with eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import synth
from gpu_util import seed_of, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_decode_step_replays_from_a_graph(variant):
    steps = 6
    wd = synth.make_decode(variant, 64, 4, 128, 128, steps=steps, in_dtype="bf16", seed=seed_of("graph", variant))
    dev = torch.device("cuda:0")

    def tok(s):
        return dict(q=to_dev(wd.q[s], "bf16"), k=to_dev(wd.k[s], "bf16"), v=to_dev(wd.v[s], "bf16"),
                    alpha=to_dev(wd.alpha[s]), erase=to_dev(wd.erase[s]),
                    write=None if wd.write is None else to_dev(wd.write[s]))

    static = tok(0)
    S0 = to_dev(wd.S0)
    S_g = S0.clone()
    o_g = torch.empty((64, 4, 128), dtype=torch.float32, device=dev)

    # a first call outside the capture (library load, kernel code objects)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        scratch = S0.clone()
        drl.dr_decode_step(**static, variant=variant, S=scratch, o=torch.empty_like(o_g))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        drl.dr_decode_step(**static, variant=variant, S=S_g, o=o_g)
    torch.cuda.synchronize()

    S_g.copy_(S0)  # capture runs nothing; start the replays from S0
    S_e = S0.clone()
    for s in range(steps):
        inp = tok(s)
        for name, t in inp.items():
            if t is not None:
                static[name].copy_(t)
        graph.replay()
        torch.cuda.synchronize()
        o_e = drl.decode_step(**inp, variant=variant, S=S_e)  # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {s}: output differs from the eager step"
        assert torch.equal(S_g, S_e), f"replay {s}: state differs from the eager step"
    print(f"[graph decode {variant}] {steps} replays bit-identical to eager steps", flush=True)


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_replays_from_a_graph(packed):
    # the prefill's workspace is taken and released stream-ordered, which a capture records
    # as graph memory nodes; the packed call's plan pass is captured with it
    from gpu_util import prefill_inputs
    if packed:
        wl = synth.make_prefill("rda", 1, 0, 2, 128, 128, in_dtype="bf16", seed=seed_of("graph pf", 1),
                                lengths=[70, 0, 130, 64])
    else:
        wl = synth.make_prefill("kda", 2, 150, 2, 128, 128, in_dtype="bf16", seed=seed_of("graph pf", 0))
    a = prefill_inputs(wl)
    B, T, H, _ = wl.q.shape
    dev = torch.device("cuda:0")
    o_g = torch.empty((B, T, H, 128), device=dev)
    S_g = torch.empty((wl.S0.shape[0], H, 128, 128), device=dev)

    def call(o, S):
        drl.dr_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], a["variant"], a["S0"],
                         a["cu_seqlens"], o, S)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(torch.empty_like(o_g), torch.empty_like(S_g))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o_g, S_g)
    torch.cuda.synchronize()
    for r in range(4):
        o_g.zero_()
        S_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        o_e, S_e = torch.empty_like(o_g), torch.empty_like(S_g)
        call(o_e, S_e)  # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e), f"replay {r} differs from the eager call"
    print(f"[graph prefill packed={packed}] 4 replays bit-identical to eager calls", flush=True)


def test_noalloc_strided_windowed_prefill_replays_from_a_graph(monkeypatch):
    # the allocation-free prefill (its workspace the library's static scratch: no memory nodes),
    # on q, k, v given as views of one fused projection, in windows of two chunks; eager calls
    # of the same entry point share the scratch between the replays
    from gpu_util import prefill_inputs
    monkeypatch.setenv("DR_WINDOW_BYTES", str(2 * 2 * 2 * 132 * 1024))  # two chunks of 2 rows x 2 heads
    wl = synth.make_prefill("kda", 2, 300, 2, 128, 128, in_dtype="bf16", seed=seed_of("graph noalloc"))
    a = prefill_inputs(wl)
    plan = drl.chunk_fwd_plan_ex(2, 300, 2, 128, 128, noalloc=True)
    assert plan["windows"] == 3 and plan["window_chunks"] == 2, plan
    fused = torch.stack([a["q"], a["k"], a["v"]], dim=2).contiguous()
    q, k, v = fused[:, :, 0], fused[:, :, 1], fused[:, :, 2]
    B, T, H, _ = wl.q.shape
    o_g = torch.empty((B, T, H, 128), device=q.device)
    S_g = torch.empty((B, H, 128, 128), device=q.device)

    def call(o, S):
        drl.dr_chunk_fwd_noalloc(q, k, v, a["alpha"], a["erase"], None, "kda", a["S0"], None, o, S)

    o_ref, S_ref = torch.empty_like(o_g), torch.empty_like(S_g)
    drl.dr_chunk_fwd_ex(a["q"], a["k"], a["v"], a["alpha"], a["erase"], None, "kda", a["S0"], None, o_ref, S_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(torch.empty_like(o_g), torch.empty_like(S_g))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o_g, S_g)
    torch.cuda.synchronize()
    for r in range(4):
        o_g.zero_()
        S_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(S_g, S_ref), f"replay {r} differs from the pooled call"
        o_e, S_e = torch.empty_like(o_g), torch.empty_like(S_g)
        call(o_e, S_e)  # eager, on the same scratch, between the replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_ref) and torch.equal(S_e, S_ref)
    print("[graph noalloc strided windows] 4 replays bit-identical to the pooled dense call", flush=True)
