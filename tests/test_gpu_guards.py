"""GPU: guard bands around every output buffer. Each output lives inside a larger allocation whose
leading and trailing guard regions hold a NaN bit pattern; after the call the guards must be
unchanged bit for bit (no kernel writes outside its outputs), for every prefill layout and option,
the decode step and the backward pass."""
import math

import pytest
import torch

import delta_rule_linear_chunked_amd as drl
import synth
from gpu_util import decode_inputs, prefill_inputs, seed_of, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096              # elements on each side (16 KiB for fp32: keeps 16-byte alignment)
SENTINEL = 0x7FC0DEAD     # a quiet NaN with a payload no kernel produces


class Guarded:
    """An fp32 tensor of `shape` inside a larger buffer with guard bands on both sides."""

    def __init__(self, shape, fill=None):
        self.n = math.prod(shape)
        self.big = torch.empty(self.n + 2 * GUARD, dtype=torch.float32, device="cuda:0")
        self.big.view(torch.int32).fill_(SENTINEL)
        self.t = self.big[GUARD:GUARD + self.n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self):
        b = self.big.view(torch.int32)
        return bool((b[:GUARD] == SENTINEL).all()) and bool((b[GUARD + self.n:] == SENTINEL).all())


def _prefill(a, N, H, dk, dv, variant, **kw):
    B, T = a["q"].shape[:2]
    o, S = Guarded((B, T, H, dv)), Guarded((N, H, dk, dv))
    drl.dr_chunk_fwd_ex(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], variant, a["S0"],
                        a["cu_seqlens"], o.t, S.t, **kw)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("case", ["fixed", "packed", "windows", "product2"])
def test_prefill_writes_only_its_outputs(case, monkeypatch):
    if case == "packed":
        wl = synth.make_prefill("gdn2", 1, 0, 3, 64, 32, in_dtype="bf16", seed=seed_of("guard", case),
                                lengths=[65, 0, 1, 130, 63])
    elif case == "product2":
        wl = synth.make_product("kda", 2, 77, 2, 64, 64, in_dtype="bf16", seed=seed_of("guard", case))
    else:
        if case == "windows":
            monkeypatch.setenv("DR_WINDOW_BYTES", "1")  # one chunk of every sequence per window
        wl = synth.make_prefill("ckda", 3, 150, 2, 128, 128, in_dtype="bf16", seed=seed_of("guard", case))
    a = prefill_inputs(wl)
    B, T, H, dk = a["q"].shape
    dv = a["v"].shape[-1]
    N = wl.S0.shape[0]
    o, S = _prefill(a, N, H, dk, dv, wl.variant)
    assert o.intact() and S.intact(), case
    assert torch.isfinite(o.t).all() and torch.isfinite(S.t).all()


def test_stored_states_and_pools_write_only_their_rows(monkeypatch):
    wl = synth.make_prefill("kda", 2, 200, 2, 64, 64, in_dtype="bf16", seed=seed_of("guard states"))
    a = prefill_inputs(wl)
    B, T, H, dk = a["q"].shape
    for window_bytes in (None, "1"):
        if window_bytes:
            monkeypatch.setenv("DR_WINDOW_BYTES", window_bytes)
        # snapshots every 64 tokens: 3 rows per sequence
        snaps = Guarded((B * (T // 64), H, dk, 64))
        o, S = _prefill(a, B, H, dk, 64, "kda", snapshots=snaps.t, snapshot_every=64)
        assert snaps.intact() and o.intact() and S.intact()
        # a pool of 5 slots; sequence 1 outside the pool (no state read or written)
        pool = Guarded((5, H, dk, 64), fill=torch.randn((5, H, dk, 64), device="cuda:0"))
        before = pool.t.clone()
        idx = torch.tensor([3, -1], dtype=torch.int32, device="cuda:0")
        o2 = Guarded((B, T, H, 64))
        drl.dr_chunk_fwd_ex(a["q"], a["k"], a["v"], a["alpha"], a["erase"], None, "kda", pool.t, None, o2.t, pool.t,
                            state_idx=idx)
        torch.cuda.synchronize()
        assert pool.intact() and o2.intact()
        keep = [0, 1, 2, 4]
        assert torch.equal(pool.t[keep], before[keep])  # only slot 3 changes


def test_noalloc_writes_only_its_outputs():
    wl = synth.make_prefill("rda", 1, 0, 2, 128, 64, in_dtype="bf16", seed=seed_of("guard noalloc"),
                            lengths=[100, 3, 0, 64])
    a = prefill_inputs(wl)
    B, T, H, dk = a["q"].shape
    o, S = Guarded((B, T, H, 64)), Guarded((4, H, dk, 64))
    drl.dr_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], "rda", a["S0"],
                             a["cu_seqlens"], o.t, S.t)
    torch.cuda.synchronize()
    assert o.intact() and S.intact()


@pytest.mark.parametrize("variant", ["kda", "gdn2", "product2"])
def test_decode_writes_only_its_outputs(variant):
    if variant == "product2":
        wl = synth.make_product_decode("kda", 7, 3, 64, 64, steps=1, in_dtype="bf16", seed=seed_of("guard dec p2"))
    else:
        wl = synth.make_decode(variant, 7, 3, 128, 64, steps=1, in_dtype="bf16", seed=seed_of("guard dec", variant))
    a = decode_inputs(wl, 0)
    N, H, dk = a["q"].shape
    dv = a["v"].shape[-1]
    S = Guarded((N, H, dk, dv), fill=to_dev(wl.S0))
    o = Guarded((N, H, dv))
    drl.dr_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], a["variant"], S.t, o.t)
    torch.cuda.synchronize()
    assert S.intact() and o.intact()
    # through a slot pool, one sequence outside it
    pool = Guarded((N + 2, H, dk, dv), fill=torch.randn((N + 2, H, dk, dv), device="cuda:0"))
    idx = torch.tensor(list(range(N - 1)) + [-1], dtype=torch.int32, device="cuda:0")
    o2 = Guarded((N, H, dv))
    drl.dr_decode_step_ex(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], a["variant"], pool.t, o2.t,
                          state_idx=idx)
    torch.cuda.synchronize()
    assert pool.intact() and o2.intact()


@pytest.mark.parametrize("variant,packed", [("kda", False), ("gdn2", True), ("rda", False)])
def test_backward_writes_only_its_gradients(variant, packed):
    if packed:
        wl = synth.make_prefill(variant, 1, 0, 2, 64, 64, in_dtype="bf16", seed=seed_of("guard bwd", variant),
                                lengths=[70, 1, 0, 64])
    else:
        wl = synth.make_prefill(variant, 2, 130, 2, 64, 64, in_dtype="bf16", seed=seed_of("guard bwd", variant))
    a = prefill_inputs(wl)
    B, T, H, dk = a["q"].shape
    dv = a["v"].shape[-1]
    N = wl.S0.shape[0]
    dO = torch.randn((B, T, H, dv), device="cuda:0")
    g = {name: Guarded(shape) for name, shape in (("dq", (B, T, H, dk)), ("dk", (B, T, H, dk)), ("dv", (B, T, H, dv)),
                                                  ("dalpha", (B, T, H, dk)), ("dS0", (N, H, dk, dv)))}
    g["derase"] = Guarded(tuple(a["erase"].shape))
    g["dwrite"] = None if a["write"] is None else Guarded(tuple(a["write"].shape))
    drl.dr_chunk_bwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], variant, a["S0"], a["cu_seqlens"],
                     dO, None, g["dq"].t, g["dk"].t, g["dv"].t, g["dalpha"].t, g["derase"].t,
                     None if g["dwrite"] is None else g["dwrite"].t, g["dS0"].t)
    torch.cuda.synchronize()
    for name, x in g.items():
        if x is not None:
            assert x.intact(), name
