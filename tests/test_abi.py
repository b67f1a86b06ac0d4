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
    assert lib.dr_version() >= 100


FAKE = ctypes.c_void_p(0x100000)       # 16-byte aligned, never dereferenced: every call below
MISALIGNED = ctypes.c_void_p(0x100004)  # fails validation before any HIP call


def dims(B=1, T=8, H=2, dk=64, dv=64, N=None, dt=1, reserved=0):
    return drl._Dims(B, T, H, dk, dv, B if N is None else N, dt, reserved)


def chunk(lib, d, variant=0, write=None, S0=None, cu=None, q=FAKE, o=FAKE):
    return lib.dr_chunk_fwd(q, FAKE, FAKE, FAKE, FAKE, write, variant, S0, cu, o, None,
                            ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("case,expect", [
    (dict(d=None), -1),
    (dict(d=dims(dk=48)), -5),
    (dict(d=dims(dv=256)), -5),
    (dict(d=dims(dt=7)), -3),
    (dict(d=dims(reserved=1)), -2),
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
