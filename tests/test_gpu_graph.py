"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): the step allocates
nothing and never synchronises, so a serving loop can replay it. Each replay is checked
against the same step run eagerly (same kernel, same inputs: bit-identical), with eager work
and synchronisations between the replays."""
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
