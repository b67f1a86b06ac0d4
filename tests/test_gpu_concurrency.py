"""GPU: calls from several host threads at once, each on its own stream. The library's host state
(the per-device workspace pool, created under a lock, and the thread-local error message) and its
stream-ordered workspace must keep the calls apart: every result equals the same call made alone
on the default stream, bit for bit. (dr_chunk_fwd_noalloc is left out: its calls share one static
scratch per GPU and are documented to race when they overlap.)"""
import threading

import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import synth
from gpu_util import decode_inputs, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu


def _cases():
    return [
        ("kda", synth.make_prefill("kda", 2, 700, 4, 128, 128, in_dtype="bf16", seed=seed_of("conc", 0))),
        ("gdn2", synth.make_prefill("gdn2", 1, 0, 3, 64, 64, in_dtype="bf16", seed=seed_of("conc", 1),
                                    lengths=[300, 0, 1, 130])),
        ("rda", synth.make_prefill("rda", 3, 257, 2, 64, 32, in_dtype="f32", seed=seed_of("conc", 2))),
        ("ckda", synth.make_prefill("ckda", 1, 1000, 2, 128, 64, in_dtype="bf16", seed=seed_of("conc", 3))),
    ]


def _run(a, dec, S_dec):
    o, S_T = drl.chunk_fwd(**a)
    S = S_dec.clone()
    od = drl.decode_step(S=S, **dec)
    return o, S_T, od, S


def test_threads_on_their_own_streams():
    cases = _cases()
    inputs = []
    for i, (name, wl) in enumerate(cases):
        dwl = synth.make_decode(name, 5, 2, wl.q.shape[3], wl.v.shape[3], steps=1, in_dtype=wl.in_dtype,
                                seed=seed_of("conc dec", i))
        inputs.append((prefill_inputs(wl), decode_inputs(dwl, 0), to_dev(dwl.S0)))
    ref = [_run(*x) for x in inputs]
    torch.cuda.synchronize()

    results = [[None] * 4 for _ in cases]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(4):
                    results[i][rep] = _run(*inputs[i])
            s.synchronize()
        except Exception as e:  # reported below, on the test's thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (name, _) in enumerate(cases):
        for rep in range(4):
            for got, want in zip(results[i][rep], ref[i]):
                assert torch.equal(got, want), (name, rep)
