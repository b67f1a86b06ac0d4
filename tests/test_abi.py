"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

import delta_rule_linear_chunked_amd as drl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltarule.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(drl.library_path()):
        from delta_rule_linear_chunked_amd import _build
        _build.build(verbose=False)
    return drl.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dr_chunk_fwd", "dr_decode_step", "dr_status_string", "dr_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, -8, -1):
        assert lib.dr_status_string(code).decode().startswith("DR_")
    assert lib.dr_status_string(-4).decode().startswith("DR_ERR_LAYOUT")
    assert lib.dr_version() >= 100


FAKE = ctypes.c_void_p(0x100000)       # 16-byte aligned, never dereferenced: every call below
MISALIGNED = ctypes.c_void_p(0x100004)  # fails validation before any HIP call


def dims(B=1, T=8, H=2, dk=64, dv=64, N=None, dt=1, version=0):
    return drl._Dims(B, T, H, dk, dv, B if N is None else N, dt, version)


def chunk(lib, d, variant=0, write=None, S0=None, cu=None, q=FAKE, o=FAKE):
    return lib.dr_chunk_fwd(q, FAKE, FAKE, FAKE, FAKE, write, variant, S0, cu, o, None,
                            ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("case,expect", [
    (dict(d=None), -1),
    (dict(d=dims(dk=48)), -5),
    (dict(d=dims(dv=256)), -5),
    (dict(d=dims(dt=7)), -3),
    (dict(d=dims(version=1)), -2),
    (dict(d=dims(T=-1)), -2),
    (dict(d=dims(H=0)), -2),
    (dict(d=dims(), variant=9), -6),
    (dict(d=dims(), variant=0, write=FAKE), -6),     # KDA takes no write gate
    (dict(d=dims(), variant=3, write=FAKE), -6),     # CKDA neither
    (dict(d=dims(), variant=4, write=FAKE), -6),     # nor the two-transition variant
    (dict(d=dims(), variant=1, write=None), -6),     # RDA needs one
    (dict(d=dims(), variant=2, write=None), -6),     # GDN-2 needs one
    (dict(d=dims(B=2, N=3)), -2),                    # N must equal B without cu_seqlens
    (dict(d=dims(B=2, N=3), cu=FAKE), -2),           # packed needs B == 1
    (dict(d=dims(), q=None), -1),
    (dict(d=dims(), o=MISALIGNED), -4),             # o is optional (states only), but aligned
    (dict(d=dims(), q=MISALIGNED), -4),
    (dict(d=dims(), S0=MISALIGNED), -4),
    # 2^27 sequences x 15 heads pass the 32-bit count checks, but the state pass would need
    # more than 2^31 - 1 workgroups
    (dict(d=dims(B=1, T=1 << 28, H=15, dk=128, dv=128, N=1 << 27), cu=FAKE), -5),
])
def test_chunk_fwd_rejects_bad_arguments(lib, case, expect):
    st = chunk(lib, **case)
    assert st == expect, lib.dr_last_error()
    assert lib.dr_last_error().decode() != ""


def test_decode_rejects_bad_arguments(lib):
    d = dims(T=1)
    st = lib.dr_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, FAKE, ctypes.byref(d), None)
    assert st == -6
    st = lib.dr_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, ctypes.byref(d), None)
    assert st == -1
    d = dims(T=1, dk=8)
    st = lib.dr_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, ctypes.byref(d), None)
    assert st == -5


def test_empty_problems_launch_nothing(lib):
    # no sequences: nothing to do, success without touching the device
    assert chunk(lib, dims(B=0, T=5)) == 0
    d = dims(B=0, T=1)
    assert lib.dr_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, ctypes.byref(d), None) == 0


def test_plan(lib):
    # 64 (sequence, head) pairs of d = 128: four 32-wide value blocks fill the 256 CUs
    c, b, w = drl.chunk_fwd_plan(4, 4096, 16, 128, 128)
    assert (c, b, w) == (64, 32, 256)
    # too few pairs for 32-wide blocks to fill the chip: 16-wide blocks
    assert drl.chunk_fwd_plan(1, 4096, 16, 128, 128)[1:] == (16, 128)
    # 192 pairs: 32-wide blocks already give 768 workgroups
    assert drl.chunk_fwd_plan(1, 32768, 16, 128, 128, num_seqs=12) == (64, 32, 768)
    # grid padded to a multiple of the 8 XCDs
    assert drl.chunk_fwd_plan(1, 64, 2, 16, 16)[2] == 8


def _opts(state_idx=None, num_slots=0, snapshots=None, every=0, **prep):
    o = drl._Opts(state_idx, num_slots, snapshots, every)
    for k, v in prep.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("opts,expect", [
    (dict(snapshots=0x100000, every=100), -2),         # stride not a multiple of 64
    (dict(snapshots=0x100000, every=0), -2),
    (dict(snapshots=0x100004, every=64), -4),          # misaligned snapshot buffer
    (dict(state_idx=0x100004, num_slots=4), -4),       # misaligned slot table
    (dict(state_idx=0x100000, num_slots=-1), -2),
    (dict(alpha_dtype=7), -3),                          # alpha neither fp32 nor bf16
    (dict(alpha_act=3), -5),                           # sigmoid is not a decay activation
    (dict(gate_act=1), -5),                            # nor softplus-decay a gate one
    (dict(l2norm_qk=2), -5),
    (dict(alpha_act=1, alpha_scale=float("inf")), -5),
])
def test_state_options_are_checked(lib, opts, expect):
    o = _opts(**opts)
    st = lib.dr_chunk_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, FAKE, None,
                             ctypes.byref(dims()), ctypes.byref(o), None)
    assert st == expect, lib.dr_last_error()


def test_two_transition_variant_options(lib):
    # snapshots count tokens: a multiple of 32 tokens is a multiple of 64 steps
    o = _opts(snapshots=0x100000, every=48)
    st = lib.dr_chunk_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, None, None, FAKE, None,
                             ctypes.byref(dims()), ctypes.byref(o), None)
    assert st == -2, lib.dr_last_error()
    assert "multiple of 32" in lib.dr_last_error().decode()
    # its beta is one gate for both uses: no separate write gradient
    st = lib.dr_chunk_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, None, None, FAKE, None,
                          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(dims()), None)
    assert st == -6, lib.dr_last_error()


def test_decode_takes_no_snapshots(lib):
    o = _opts(snapshots=0x100000, every=64)
    d = dims(T=1)
    st = lib.dr_decode_step_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, ctypes.byref(d),
                               ctypes.byref(o), None)
    assert st == -2, lib.dr_last_error()


def test_backward_checkpoints_are_checked(lib):
    # a misaligned checkpoint buffer is rejected before anything runs
    st = lib.dr_chunk_bwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, FAKE, None,
                             FAKE, FAKE, FAKE, FAKE, FAKE, None, None, MISALIGNED, ctypes.byref(dims()), None)
    assert st == -4, lib.dr_last_error()
    assert "checkpoints" in lib.dr_last_error().decode()


# ----------------------------------------------------------------- the binding's host checks
# (CPU tensors: every case below raises in the binding before the library is called)
def _cpu_prefill(B=1, T=130, H=2, d=64):
    import torch
    z = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    return dict(q=z(B, T, H, d), k=z(B, T, H, d), v=z(B, T, H, d), alpha=z(B, T, H, d), erase=z(B, T, H),
                write=None, variant="kda", S0=None)


def test_binding_checks_offsets():
    import torch
    T = 130
    assert drl.check_offsets(torch.tensor([0, 50, 50, 130], dtype=torch.int32), T) == [50, 0, 80]
    assert drl.check_offsets(torch.tensor([0, 64], dtype=torch.int32), T) == [64]   # rows past the end
    for bad, msg in (([1, 50, 130], "start at 0"), ([0, 80, 50, 130], "decreases"), ([0, 70, 131], "past")):
        with pytest.raises(ValueError, match=msg):
            drl.check_offsets(torch.tensor(bad, dtype=torch.int32), T)
    a = _cpu_prefill(T=T)
    with pytest.raises(ValueError, match="decreases"):
        drl.chunk_fwd(**a, cu_seqlens=torch.tensor([0, 80, 50, 130], dtype=torch.int32))


def test_binding_checks_snapshot_rows():
    import torch
    a = _cpu_prefill(B=2, T=130)
    o = torch.empty(2, 130, 2, 64)
    # fixed length: floor(130 / 64) = 2 rows per sequence, 4 in all
    for rows in (3, 5):
        snaps = torch.empty(rows, 2, 64, 64)
        with pytest.raises(ValueError, match="snapshots has shape"):
            drl.dr_chunk_fwd_ex(a["q"], a["k"], a["v"], a["alpha"], a["erase"], None, "kda", None, None, o, None,
                                snapshots=snaps, snapshot_every=64)
    # packed: rows from the host copy of the offsets (64 + 66 -> 1 + 1)
    p = _cpu_prefill(B=1, T=130)
    cu = torch.tensor([0, 64, 130], dtype=torch.int32)
    with pytest.raises(ValueError, match="snapshots has shape"):
        drl.dr_chunk_fwd_ex(p["q"], p["k"], p["v"], p["alpha"], p["erase"], None, "kda", None, cu,
                            torch.empty(1, 130, 2, 64), None, snapshots=torch.empty(1, 2, 64, 64),
                            snapshot_every=64)
    with pytest.raises(ValueError, match="decreases"):
        drl.dr_chunk_fwd_ex(p["q"], p["k"], p["v"], p["alpha"], p["erase"], None, "kda", None,
                            torch.tensor([0, 90, 40, 130], dtype=torch.int32), torch.empty(1, 130, 2, 64), None,
                            snapshots=torch.empty(1, 2, 64, 64), snapshot_every=64)
    # the backward's checkpoints: floor(len / 64) rows per sequence as well
    with pytest.raises(ValueError, match="checkpoints has shape"):
        drl.chunk_bwd(**{k: v for k, v in a.items() if k != "variant"}, variant="kda",
                      dO=torch.zeros(2, 130, 2, 64), checkpoints=torch.empty(3, 2, 64, 64))


def test_window_plans_bound_the_workspace(monkeypatch):
    monkeypatch.delenv("DR_WINDOW_BYTES", raising=False)
    # the KDA prefill workload (B=4, T=4096, H=16, d=128) needs 526 MB of records in all and runs
    # as one window under the 1 GiB default budget
    pl = drl.chunk_fwd_plan_ex(4, 4096, 16, 128, 128)
    assert pl["windows"] == 1 and pl["window_chunks"] == 64 and pl["workspace"] < 2 ** 30, pl
    # a 1M-token, 32-head sequence (69 GB of records as one window) runs in windows within 1 GiB
    # plus the carried state (32 x 128 x 128 x 4 bytes)
    pl = drl.chunk_fwd_plan_ex(1, 2 ** 20, 32, 128, 128)
    assert pl["windows"] > 1 and pl["workspace"] <= 2 ** 30 + 32 * 128 * 128 * 4, pl
    # the allocation-free plan of that sequence fits its static scratch
    pl = drl.chunk_fwd_plan_ex(1, 2 ** 20, 32, 128, 128, noalloc=True)
    assert pl["workspace"] <= drl.NOALLOC_SCRATCH_BYTES, pl
    # packed sequences run as one window
    pl = drl.chunk_fwd_plan_ex(1, 32768, 16, 128, 128, num_seqs=12)
    assert pl["windows"] == 1 and pl["window_chunks"] == 0, pl
    # under a smaller budget the KDA workload takes four windows of 16 chunks
    monkeypatch.setenv("DR_WINDOW_BYTES", str(144 * 2 ** 20))
    pl = drl.chunk_fwd_plan_ex(4, 4096, 16, 128, 128)
    assert pl["windows"] == 4 and pl["window_chunks"] == 16, pl


def _v2(strides, **kw):
    d = dims(**kw)
    d.version = drl.DIMS_V2
    return drl._DimsV2(d, *strides)


def _v2_ptr(d2):
    return ctypes.cast(ctypes.pointer(d2), ctypes.POINTER(drl._Dims))


@pytest.mark.parametrize("strides,expect", [
    ((3 * 2 * 64, 8 * 3 * 2 * 64) * 3, 0),       # views of one [1, 8, 3, H, d] projection
    ((-128, 1024, 128, 1024, 128, 1024), -2),     # negative stride
    ((132, 1056, 128, 1024, 128, 1024), -4),      # 132 bf16 elements: not a multiple of 16 bytes
    ((128, 1024, 128, 1024, 128, 1 << 41), -4),   # beyond 2^40
])
def test_strided_dims_are_checked(lib, strides, expect):
    # empty problem (B = 0) when the strides are valid: the call returns before any launch
    d2 = _v2(strides, B=0 if expect == 0 else 1, T=8)
    st = lib.dr_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, FAKE, None, _v2_ptr(d2), None)
    assert st == expect, lib.dr_last_error()


def test_backward_checks_strides(lib):
    dq = FAKE
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, FAKE, None, dq, FAKE, FAKE, FAKE, FAKE, None, None]
    # views of one [B, T, 3, H, d] projection are accepted (B = 0: the call returns before any
    # launch); a stride that is not a multiple of 16 bytes is a layout error, as for the forward
    strided = _v2((384, 3072, 384, 3072, 384, 3072), B=0, T=8)
    strided.base.num_seqs = 0
    assert lib.dr_chunk_bwd(*args, _v2_ptr(strided), None) == 0, lib.dr_last_error()
    bad = _v2((132, 1056, 128, 1024, 128, 1024), B=2, T=8)
    assert lib.dr_chunk_bwd(*args, _v2_ptr(bad), None) == -4  # DR_ERR_LAYOUT


def test_unknown_dims_version_is_rejected(lib):
    assert chunk(lib, dims(version=3)) == -2


def test_last_error_is_per_thread(lib):
    # dr_last_error() is thread-local: threads making failing calls at the same time (ctypes
    # releases the GIL around each call) each read back the message of their own call
    import threading

    errors = []

    def worker(i):
        dk = 17 + i                                   # unsupported, and different in every thread
        for _ in range(300):
            st = chunk(lib, dims(dk=dk))
            msg = lib.dr_last_error().decode()
            if st != -5 or f"d_k={dk} " not in msg:
                errors.append((i, st, msg))
                return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
