"""Helpers for the GPU parity tests: move a synthetic workload to the device, run the
HIP path through the binding, and run the fp64 oracle on all or on a sample of the
(sequence, head) pairs. The oracle sees exactly the values handed to the GPU."""
from __future__ import annotations

import zlib

import numpy as np
import torch

import delta_rule_linear_chunked_amd as drl
import oracle

TOL = {"f32": 1e-4, "bf16": 1e-2}


def seed_of(*parts) -> int:
    """A seed fixed by the test's parameters (Python's own hash() of strings changes from
    one process to the next)."""
    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def device():
    return torch.device("cuda:0")


def to_dev(x, in_dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x)).to(device())
    if in_dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def prefill_inputs(wl):
    return dict(q=to_dev(wl.q, wl.in_dtype), k=to_dev(wl.k, wl.in_dtype), v=to_dev(wl.v, wl.in_dtype),
                alpha=to_dev(wl.alpha), erase=to_dev(wl.erase), write=to_dev(wl.write),
                variant=wl.variant, S0=to_dev(wl.S0),
                cu_seqlens=None if wl.cu_seqlens is None else to_dev(wl.cu_seqlens))


def run_prefill(wl, S0_override="keep"):
    a = prefill_inputs(wl)
    if S0_override != "keep":
        a["S0"] = S0_override
    o, S_T = drl.chunk_fwd(**a)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), S_T.cpu().numpy().astype(np.float64)


def _gate(x, sl):
    return None if x is None else x[sl]


def oracle_prefill(wl, pairs=None):
    """Oracle (o, S_T). With ``pairs`` (list of (sequence, head)), only those pairs are
    computed; results come back as o_pairs [P][T_n, dv] and S_pairs [P, dk, dv]."""
    if pairs is None:
        return oracle.step_recurrence(wl.q, wl.k, wl.v, wl.alpha, wl.erase, wl.write, wl.variant,
                                      S0=wl.S0, cu_seqlens=wl.cu_seqlens)
    outs, states = [], []
    for (n, h) in pairs:
        if wl.cu_seqlens is None:
            sl = (slice(n, n + 1), slice(None), slice(h, h + 1))
        else:
            t0, t1 = int(wl.cu_seqlens[n]), int(wl.cu_seqlens[n + 1])
            sl = (slice(0, 1), slice(t0, t1), slice(h, h + 1))
        S0 = None if wl.S0 is None else wl.S0[n:n + 1, h:h + 1]
        o, S = oracle.step_recurrence(wl.q[sl], wl.k[sl], wl.v[sl], wl.alpha[sl], _gate(wl.erase, sl),
                                      _gate(wl.write, sl), wl.variant, S0=S0)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return outs, np.stack(states)


def gpu_pairs(wl, o, S_T, pairs):
    outs = []
    for (n, h) in pairs:
        if wl.cu_seqlens is None:
            outs.append(o[n, :, h])
        else:
            t0, t1 = int(wl.cu_seqlens[n]), int(wl.cu_seqlens[n + 1])
            outs.append(o[0, t0:t1, h])
    return outs, np.stack([S_T[n, h] for (n, h) in pairs])


def decode_inputs(wl, step):
    t = step
    return dict(q=to_dev(wl.q[t], wl.in_dtype), k=to_dev(wl.k[t], wl.in_dtype), v=to_dev(wl.v[t], wl.in_dtype),
                alpha=to_dev(wl.alpha[t]), erase=to_dev(wl.erase[t]),
                write=None if wl.write is None else to_dev(wl.write[t]), variant=wl.variant)
