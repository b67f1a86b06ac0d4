"""The allocation-free prefill entry point (dr_chunk_fwd_noalloc), through the C ABI, against the
entry point it mirrors (dr_chunk_fwd_ex, whose workspace comes from the library's pool).

Two calls in a row, the second on a smaller problem, so the second runs on what the first left in
the static scratch; both must equal the pooled call bit for bit (the same kernels run on the same
inputs) and match the fp64 oracle within the parity bar. Fixed-length problems whose records would
not fit run in more, shorter windows of chunk positions and still equal the pooled call bit for bit;
packed sequences (one window) whose workspace exceeds the scratch are rejected before anything is
launched."""
import numpy as np
import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import oracle
import synth
from gpu_util import TOL, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _both(wl):
    a = prefill_inputs(wl)
    B, T, H, _ = a["q"].shape
    N = wl.S0.shape[0]
    dv = a["v"].shape[-1]
    dk = a["q"].shape[-1]
    outs = []
    for entry in (drl.dr_chunk_fwd_ex, drl.dr_chunk_fwd_noalloc):
        o = torch.full((B, T, H, dv), 7.0, dtype=torch.float32, device=a["q"].device)
        S = torch.full((N, H, dk, dv), 7.0, dtype=torch.float32, device=a["q"].device)
        entry(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], wl.variant, a["S0"], a["cu_seqlens"], o, S)
        outs.append((o, S))
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_the_pooled_entry_point_on_two_calls():
    big = synth.make_prefill("ckda", 2, 1000, 4, 128, 128, in_dtype="bf16", seed=seed_of("noalloc", 1))
    small = synth.make_prefill("gdn2", 1, 0, 3, 64, 64, in_dtype="bf16", seed=seed_of("noalloc", 2),
                               lengths=[70, 0, 130, 5])
    for wl in (big, small):
        (o_ref, S_ref), (o, S) = _both(wl)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), wl.name
        oo, so = oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant, S0=wl.S0,
                                        cu_seqlens=wl.cu_seqlens)
        eo = oracle.rel_err(o.cpu().numpy(), oo)
        es = oracle.rel_err(S.cpu().numpy(), so)
        print(f"[noalloc {wl.name}] err o={eo:.3e} S_T={es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


def test_noalloc_runs_a_long_fixed_length_problem_in_windows():
    # 16384 tokens x 16 heads at d = 128: about 526 MB of records as one window; in windows of
    # chunk positions the workspace fits the scratch
    wl = synth.make_prefill("kda", 1, 16384, 16, 128, 128, in_dtype="bf16", seed=seed_of("noalloc", 3))
    plan = drl.chunk_fwd_plan_ex(1, 16384, 16, 128, 128, variant="kda", noalloc=True)
    assert plan["windows"] > 1 and plan["workspace"] <= drl.NOALLOC_SCRATCH_BYTES, plan
    (o_ref, S_ref), (o, S) = _both(wl)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # two packed sequences of 8192 tokens x 16 heads at d = 128: packed sequences run as one
    # window, about 526 MB of workspace
    B, T, H, d = 1, 16384, 16, 128
    dev = torch.device("cuda:0")
    q = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device=dev)
    alpha = torch.ones((B, T, H, d), dtype=torch.float32, device=dev)
    beta = torch.zeros((B, T, H), dtype=torch.float32, device=dev)
    cu = torch.tensor([0, 8192, 16384], dtype=torch.int32, device=dev)
    o = torch.full((B, T, H, d), 7.0, dtype=torch.float32, device=dev)
    plan = drl.chunk_fwd_plan_ex(1, 16384, 16, 128, 128, num_seqs=2, variant="kda", noalloc=True)
    assert plan["workspace"] > drl.NOALLOC_SCRATCH_BYTES, plan
    with pytest.raises(drl.DeltaRuleError, match="DR_ERR_UNSUPPORTED"):
        drl.dr_chunk_fwd_noalloc(q, q, q, alpha, beta, None, "kda", None, cu, o, None)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
