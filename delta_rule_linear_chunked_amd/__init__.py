"""Python binding of libdeltarule (gated delta-rule prefill and decode on MI355X).

Argument marshalling only: the functions check that the torch tensors have the
shapes, dtypes and layout the C ABI expects, pass raw device pointers and the
current HIP stream, and raise on a non-zero status. Every step of the
computation runs in the HIP kernels of ``lib/libdeltarule.so``; there is no
fallback. If the library has not been built the first call raises.

The names mirror the C entry points (``dr_chunk_fwd``, ``dr_decode_step``);
``chunk_fwd`` and ``decode_step`` additionally allocate the outputs; ``delta_rule``
wires the prefill and its backward into torch autograd.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["dr_chunk_fwd", "dr_decode_step", "dr_chunk_fwd_ex", "dr_chunk_fwd_noalloc", "dr_decode_step_ex",
           "dr_chunk_bwd",
           "chunk_fwd", "delta_rule", "decode_step", "chunk_bwd", "chunk_fwd_plan", "chunk_fwd_plan_ex", "snapshot_count",
           "check_offsets",
           "library_path",
           "load_library", "VARIANTS", "DeltaRuleError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libdeltarule.so")
# "product2": two KDA transitions per token (k [.., 2, d_k], v [.., 2, d_v], beta [.., 2])
VARIANTS = {"kda": 0, "rda": 1, "gdn2": 2, "ckda": 3, "product2": 4}
_DT = {torch.float32: 0, torch.bfloat16: 1}
_lib = None
# bytes of the static device scratch behind dr_chunk_fwd_noalloc (DR_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20


class DeltaRuleError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("num_heads", ctypes.c_int64),
                ("head_dim_k", ctypes.c_int64), ("head_dim_v", ctypes.c_int64),
                ("num_seqs", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("version", ctypes.c_int32)]


DIMS_V2 = 2  # dr_dims.version of a dr_dims_v2 (strided q, k, v)


class _DimsV2(ctypes.Structure):
    _fields_ = [("base", _Dims),
                ("q_token_stride", ctypes.c_int64), ("q_batch_stride", ctypes.c_int64),
                ("k_token_stride", ctypes.c_int64), ("k_batch_stride", ctypes.c_int64),
                ("v_token_stride", ctypes.c_int64), ("v_batch_stride", ctypes.c_int64)]


class _Opts(ctypes.Structure):
    _fields_ = [("state_idx", ctypes.c_void_p), ("num_slots", ctypes.c_int64),
                ("snapshots", ctypes.c_void_p), ("snapshot_every", ctypes.c_int64),
                ("l2norm_qk", ctypes.c_int32), ("alpha_dtype", ctypes.c_int32), ("alpha_act", ctypes.c_int32),
                ("alpha_scale", ctypes.c_float), ("gate_act", ctypes.c_int32), ("gate_scale", ctypes.c_float)]


class _Plan(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("dv_block", ctypes.c_int32), ("workgroups", ctypes.c_int64),
                ("window_chunks", ctypes.c_int64), ("windows", ctypes.c_int64), ("workspace", ctypes.c_int64)]


# activations of the fused input preparation (dr_act)
ACTS = {"none": 0, "exp_neg_softplus": 1, "tanh": 2, "sigmoid": 3}


def _opts(state_idx=None, num_slots=0, snapshots=None, snapshot_every=0, prep=None, alpha=None) -> _Opts:
    """Options block; ``prep`` is a dict with l2norm_qk, alpha_act, alpha_scale, gate_act,
    gate_scale (names as in ``synth``'s pre-activation workloads); alpha's element type comes
    from the alpha tensor."""
    o = _Opts(None if state_idx is None else state_idx.data_ptr(), num_slots,
              None if snapshots is None else snapshots.data_ptr(), int(snapshot_every or 0))
    if alpha is not None and alpha.dtype == torch.bfloat16:
        o.alpha_dtype = _DT[torch.bfloat16]
    if prep:
        o.l2norm_qk = int(bool(prep.get("l2norm_qk", False)))
        o.alpha_act = ACTS[prep.get("alpha_act", "none")]
        o.alpha_scale = float(prep.get("alpha_scale", 1.0))
        o.gate_act = ACTS[prep.get("gate_act", "none")]
        o.gate_scale = float(prep.get("gate_scale", 1.0))
    return o


def _alpha_dtype(alpha, prep):
    if alpha is not None and alpha.dtype == torch.bfloat16:
        return torch.bfloat16
    return torch.float32


def library_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None):
    """Load libdeltarule.so once and declare its signatures. DELTARULE_LIBRARY in the environment
    names another build of the same library (a sanitizer build of the host code, say)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("DELTARULE_LIBRARY") or _LIB_PATH
    if not os.path.exists(p):
        raise DeltaRuleError(f"{p} is missing: build it with `python -m delta_rule_linear_chunked_amd._build`")
    lib = ctypes.CDLL(p)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    lib.dr_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, vp, fp, fp, ctypes.POINTER(_Dims), vp]
    lib.dr_chunk_fwd.restype = ip
    lib.dr_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, fp, ctypes.POINTER(_Dims), vp]
    lib.dr_decode_step.restype = ip
    op = ctypes.POINTER(_Opts)
    lib.dr_chunk_fwd_ex.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, vp, fp, fp, ctypes.POINTER(_Dims), op, vp]
    lib.dr_chunk_fwd_ex.restype = ip
    lib.dr_chunk_fwd_noalloc.argtypes = lib.dr_chunk_fwd_ex.argtypes
    lib.dr_chunk_fwd_noalloc.restype = ip
    lib.dr_decode_step_ex.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, fp, ctypes.POINTER(_Dims), op, vp]
    lib.dr_decode_step_ex.restype = ip
    lib.dr_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                 ctypes.POINTER(_Dims), vp]
    lib.dr_chunk_bwd.restype = ip
    lib.dr_chunk_bwd_ex.argtypes = [vp, vp, vp, fp, fp, fp, ip, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                    ctypes.POINTER(_Dims), vp]
    lib.dr_chunk_bwd_ex.restype = ip
    lib.dr_status_string.argtypes = [ip]
    lib.dr_status_string.restype = ctypes.c_char_p
    lib.dr_last_error.argtypes = []
    lib.dr_last_error.restype = ctypes.c_char_p
    lib.dr_version.restype = ip
    lib.dr_chunk_fwd_plan.argtypes = [ctypes.POINTER(_Dims), ip, ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    lib.dr_chunk_fwd_plan.restype = ip
    lib.dr_chunk_fwd_plan_ex.argtypes = [ctypes.POINTER(_Dims), ip, ip, ctypes.POINTER(_Plan)]
    lib.dr_chunk_fwd_plan_ex.restype = ip
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int, what: str):
    if status != 0:
        msg = lib.dr_last_error().decode()
        raise DeltaRuleError(f"{what}: {lib.dr_status_string(status).decode()}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, shape, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_rows(t: Optional[torch.Tensor], name: str, shape, nlead: int, dtype, device):
    """Check q, k or v: shape, dtype and device as ``_need``, and a layout the kernels can read
    through strides: the dimensions after the ``nlead`` leading ones (batch and token, or the
    sequence for decode) dense. Returns the element strides of the leading dimensions (0 for a
    dimension of size 1, which is never stepped over)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() == 0:  # nothing is read
        return (0,) * nlead
    inner = 1
    for dim in range(t.dim() - 1, nlead - 1, -1):
        if t.shape[dim] != 1 and t.stride(dim) != inner:
            raise ValueError(f"{name}: the dimensions after its first {nlead} must be dense (strides "
                             f"{tuple(t.stride())}); only its batch and token strides may be free")
        inner *= t.shape[dim]
    return tuple(0 if t.shape[dim] == 1 else t.stride(dim) for dim in range(nlead))


def _dims_for(B, T, H, dk, dv, N, dtype, strides):
    """dr_dims for dense q, k, v, else a dr_dims_v2 with their strides ((token, batch) x 3)."""
    d = _Dims(B, T, H, dk, dv, N, _DT[dtype], 0)
    if strides is None:
        return d
    d.version = DIMS_V2
    return _DimsV2(d, *strides)


def _dims_arg(d):
    """The pointer to pass where the C ABI takes a const dr_dims* (a dr_dims_v2 starts with one)."""
    if isinstance(d, _DimsV2):
        return ctypes.cast(ctypes.pointer(d), ctypes.POINTER(_Dims))
    return ctypes.byref(d)


def _gate_shapes(variant: str, lead, dk, dv):
    if variant in ("kda", "ckda"):
        return tuple(lead), None
    if variant == "product2":
        return tuple(lead) + (2,), None
    if variant == "rda":
        return tuple(lead), tuple(lead)
    if variant == "gdn2":
        return tuple(lead) + (dk,), tuple(lead) + (dv,)
    raise ValueError(f"unknown variant {variant!r}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd_plan(B: int, T: int, H: int, dk: int, dv: int, num_seqs: Optional[int] = None,
                   variant: str = "kda", in_dtype: torch.dtype = torch.bfloat16):
    """(chunk, dv_block, workgroups) the prefill launches for these sizes."""
    lib = load_library()
    d = _Dims(B, T, H, dk, dv, B if num_seqs is None else num_seqs, _DT[in_dtype], 0)
    c, b, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib, lib.dr_chunk_fwd_plan(ctypes.byref(d), VARIANTS[variant], ctypes.byref(c),
                                      ctypes.byref(b), ctypes.byref(w)), "dr_chunk_fwd_plan")
    return c.value, b.value, w.value


def chunk_fwd_plan_ex(B: int, T: int, H: int, dk: int, dv: int, num_seqs: Optional[int] = None,
                      variant: str = "kda", in_dtype: torch.dtype = torch.bfloat16, noalloc: bool = False) -> dict:
    """The prefill's full launch plan (dr_chunk_fwd_plan_ex) as a dict: chunk, dv_block, workgroups,
    window_chunks, windows, workspace (bytes)."""
    lib = load_library()
    d = _Dims(B, T, H, dk, dv, B if num_seqs is None else num_seqs, _DT[in_dtype], 0)
    pl = _Plan()
    _check(lib, lib.dr_chunk_fwd_plan_ex(ctypes.byref(d), VARIANTS[variant], int(noalloc), ctypes.byref(pl)),
           "dr_chunk_fwd_plan_ex")
    return {name: getattr(pl, name) for name, _ in _Plan._fields_}


def snapshot_count(lengths, every: int) -> int:
    """Rows of the snapshot buffer for sequences of these lengths: floor(len / every) each."""
    return int(sum(int(n) // int(every) for n in lengths))


def check_offsets(cu_seqlens, T: int):
    """Copy ``cu_seqlens`` to the host (a synchronisation) and check that it starts at 0, never
    decreases and ends at most at ``T``; returns the sequence lengths. Raises ValueError."""
    cu = [int(x) for x in cu_seqlens.tolist()]
    if not cu or cu[0] != 0:
        raise ValueError(f"cu_seqlens must start at 0, got {cu[:1]}")
    lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
    bad = [n for n, x in enumerate(lens) if x < 0]
    if bad:
        raise ValueError(f"cu_seqlens decreases at index {bad[0] + 1}")
    if cu[-1] > T:
        raise ValueError(f"cu_seqlens ends at {cu[-1]}, past the {T} tokens of the row")
    return lens


def _capturing() -> bool:
    return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()


def dr_chunk_fwd(q, k, v, alpha, erase, write, variant: str, S0, cu_seqlens, o, S_T) -> None:
    """Chunkwise prefill into caller-provided ``o`` (and ``S_T``). Shapes as in
    include/deltarule.h: q,k [B,T,H,dk]; v [B,T,H,dv]; alpha [B,T,H,dk] fp32; gates per
    variant (fp32); S0/S_T [N,H,dk,dv] fp32 or None; cu_seqlens [N+1] int32 or None;
    o [B,T,H,dv] fp32."""
    dr_chunk_fwd_ex(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T)


def dr_chunk_fwd_ex(q, k, v, alpha, erase, write, variant: str, S0, cu_seqlens, o, S_T,
                    state_idx=None, snapshots=None, snapshot_every: int = 0, prep=None) -> None:
    """``dr_chunk_fwd`` with options. With ``state_idx`` [N] int32, S0 and S_T are pools
    [P,H,dk,dv] whose row state_idx[n] belongs to sequence n. ``snapshots`` [num,H,dk,dv]
    fp32 receives the state after every ``snapshot_every`` tokens of each sequence (rows
    ordered by sequence, see ``snapshot_count``). ``prep`` (a dict, see ``_opts``) makes the
    kernels normalise q/k and activate alpha (fp32 or bf16) and the gates while loading."""
    _chunk_fwd_call("dr_chunk_fwd_ex", q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T,
                    state_idx, snapshots, snapshot_every, prep)


def dr_chunk_fwd_noalloc(q, k, v, alpha, erase, write, variant: str, S0, cu_seqlens, o, S_T,
                         state_idx=None, snapshots=None, snapshot_every: int = 0, prep=None) -> None:
    """``dr_chunk_fwd_ex`` with its workspace in the library's static device scratch instead of an
    allocation (for callers that cannot allocate; problems whose workspace exceeds
    ``NOALLOC_SCRATCH_BYTES`` raise). Calls that overlap on one GPU race."""
    _chunk_fwd_call("dr_chunk_fwd_noalloc", q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T,
                    state_idx, snapshots, snapshot_every, prep)


def _chunk_fwd_call(entry, q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T, state_idx, snapshots,
                    snapshot_every, prep) -> None:
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q dtype {q.dtype} is not float32 or bfloat16")
    nt = (2,) if variant == "product2" else ()  # the transition axis of k and v
    # q, k, v may be views (e.g. of one fused projection): batch and token strides are free
    sq = _need_rows(q, "q", (B, T, H, dk), 2, q.dtype, dev)
    sk = _need_rows(k, "k", (B, T, H) + nt + (dk,), 2, q.dtype, dev)
    sv = _need_rows(v, "v", (B, T, H) + nt + (dv,), 2, q.dtype, dev)
    strides = None if all(x.is_contiguous() for x in (q, k, v)) else (sq[1], sq[0], sk[1], sk[0], sv[1], sv[0])
    _need(alpha, "alpha", (B, T, H, dk), _alpha_dtype(alpha, prep), dev)
    es, ws = _gate_shapes(variant, (B, T, H), dk, dv)
    _need(erase, "erase", es, torch.float32, dev)
    if ws is None:
        if write is not None:
            raise ValueError(f"{variant} takes no write gate")
    else:
        _need(write, "write", ws, torch.float32, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    rows = N
    if state_idx is not None:
        _need(state_idx, "state_idx", (N,), torch.int32, dev)
        pools = [t for t in (S0, S_T) if t is not None]
        rows = pools[0].shape[0] if pools else 0
    if S0 is not None:
        _need(S0, "S0", (rows, H, dk, dv), torch.float32, dev)
    if S_T is not None:
        _need(S_T, "S_T", (rows, H, dk, dv), torch.float32, dev)
    if snapshots is not None:
        # rows: floor(len / every) per sequence; packed lengths need cu_seqlens on the host
        # (checked there too), which a graph capture cannot read: the row count is then the caller's
        if not snapshot_every or snapshot_every <= 0:
            raise ValueError("snapshots need a positive snapshot_every")
        if cu_seqlens is None:
            rows_s = B * (T // int(snapshot_every))
        elif not _capturing():
            rows_s = snapshot_count(check_offsets(cu_seqlens, T), snapshot_every)
        else:
            rows_s = snapshots.shape[0]
        _need(snapshots, "snapshots", (rows_s, H, dk, dv), torch.float32, dev)
    if o is not None:  # None: final states / snapshots only
        _need(o, "o", (B, T, H, dv), torch.float32, dev)
    d = _dims_for(B, T, H, dk, dv, N, q.dtype, strides)
    opts = _opts(state_idx, rows, snapshots, snapshot_every, prep, alpha)
    with torch.cuda.device(dev):  # the library launches on the current device
        st = getattr(lib, entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write),
                                 VARIANTS[variant], _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(S_T),
                                 _dims_arg(d), ctypes.byref(opts), _stream(dev))
    _check(lib, st, entry)


def dr_decode_step(q, k, v, alpha, erase, write, variant: str, S, o) -> None:
    """One decode step in place on ``S`` [N,H,dk,dv] fp32; writes ``o`` [N,H,dv] fp32.
    q,k [N,H,dk]; v [N,H,dv]; alpha [N,H,dk]; gates per variant."""
    dr_decode_step_ex(q, k, v, alpha, erase, write, variant, S, o)


def dr_decode_step_ex(q, k, v, alpha, erase, write, variant: str, S, o, state_idx=None, prep=None) -> None:
    """``dr_decode_step`` with options: with ``state_idx`` [N] int32, ``S`` is [P,H,dk,dv] and
    sequence n updates row state_idx[n] in place (a slot outside the pool: o = 0, no state);
    ``prep`` as for ``dr_chunk_fwd_ex``."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q dtype {q.dtype} is not float32 or bfloat16")
    nt = (2,) if variant == "product2" else ()
    # q, k, v may be views with a free stride between sequences
    sq = _need_rows(q, "q", (N, H, dk), 1, q.dtype, dev)[0]
    sk = _need_rows(k, "k", (N, H) + nt + (dk,), 1, q.dtype, dev)[0]
    sv = _need_rows(v, "v", (N, H) + nt + (dv,), 1, q.dtype, dev)[0]
    strides = None if all(x.is_contiguous() for x in (q, k, v)) else (0, sq, 0, sk, 0, sv)
    _need(alpha, "alpha", (N, H, dk), _alpha_dtype(alpha, prep), dev)
    es, ws = _gate_shapes(variant, (N, H), dk, dv)
    _need(erase, "erase", es, torch.float32, dev)
    if ws is None:
        if write is not None:
            raise ValueError(f"{variant} takes no write gate")
    else:
        _need(write, "write", ws, torch.float32, dev)
    rows = N
    if state_idx is not None:
        _need(state_idx, "state_idx", (N,), torch.int32, dev)
        rows = S.shape[0]
    _need(S, "S", (rows, H, dk, dv), torch.float32, dev)
    _need(o, "o", (N, H, dv), torch.float32, dev)
    d = _dims_for(N, 1, H, dk, dv, N, q.dtype, strides)
    opts = _opts(state_idx, rows, None, 0, prep, alpha)
    with torch.cuda.device(dev):
        st = lib.dr_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write),
                                   VARIANTS[variant], _ptr(S), _ptr(o), _dims_arg(d), ctypes.byref(opts),
                                   _stream(dev))
    _check(lib, st, "dr_decode_step")


def chunk_fwd(q, k, v, alpha, erase, write=None, variant: str = "kda", S0=None, cu_seqlens=None,
              output_final_state: bool = True, state_idx=None, snapshot_every: Optional[int] = None,
              prep=None, output: bool = True):
    """Allocate o (and S_T) and run the prefill. Returns (o, S_T or None), plus the snapshot
    tensor when ``snapshot_every`` is given. With ``state_idx``, S0 is a pool of states that
    is updated in place (and returned as S_T). ``output=False``: no o (None), states only."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device) if output else None
    if state_idx is not None:
        if S0 is None:
            raise ValueError("state_idx needs the pool of states as S0")
        S_T = S0
    else:
        S_T = (torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
               if output_final_state else None)
    snaps = None
    if cu_seqlens is not None and not _capturing():
        lens = check_offsets(cu_seqlens, T)
    if snapshot_every is not None:
        if cu_seqlens is None:
            lens = [T] * B
        elif _capturing():
            raise ValueError("snapshots of packed sequences need cu_seqlens on the host: not inside a graph capture")
        snaps = torch.empty((snapshot_count(lens, snapshot_every), H, dk, dv), dtype=torch.float32,
                            device=q.device)
    dr_chunk_fwd_ex(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, o, S_T, state_idx, snaps,
                    snapshot_every or 0, prep)
    return (o, S_T) if snapshot_every is None else (o, S_T, snaps)


def decode_step(q, k, v, alpha, erase, write, variant: str, S, state_idx=None, prep=None):
    """Allocate o and run the decode step (S, or its rows state_idx, updated in place).
    Returns o."""
    o = torch.empty((q.shape[0], q.shape[1], v.shape[-1]), dtype=torch.float32, device=q.device)
    dr_decode_step_ex(q, k, v, alpha, erase, write, variant, S, o, state_idx, prep)
    return o


def dr_chunk_bwd(q, k, v, alpha, erase, write, variant: str, S0, cu_seqlens, dO, dS_T,
                 dq, dk, dv, dalpha, derase, dwrite, dS0, checkpoints=None) -> None:
    """Gradients of ``dr_chunk_fwd`` into caller-provided fp32 tensors shaped like the inputs
    (dwrite None for KDA / CKDA, dS_T / dS0 optional). ``checkpoints``: the snapshots of a
    ``chunk_fwd`` on the same inputs with ``snapshot_every`` 64 (32 for product2); with them the
    call skips its own forward pass (``dr_chunk_bwd_ex``)."""
    lib = load_library()
    B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q dtype {q.dtype} is not float32 or bfloat16")
    nt = (2,) if variant == "product2" else ()  # the transition axis of k and v
    # q, k, v may be views, as for the forward: batch and token strides are free
    sq = _need_rows(q, "q", (B, T, H, dk_), 2, q.dtype, dev)
    sk = _need_rows(k, "k", (B, T, H) + nt + (dk_,), 2, q.dtype, dev)
    sv = _need_rows(v, "v", (B, T, H) + nt + (dv_,), 2, q.dtype, dev)
    strides = None if all(x.is_contiguous() for x in (q, k, v)) else (sq[1], sq[0], sk[1], sk[0], sv[1], sv[0])
    _need(alpha, "alpha", (B, T, H, dk_), torch.float32, dev)
    es, ws = _gate_shapes(variant, (B, T, H), dk_, dv_)
    _need(erase, "erase", es, torch.float32, dev)
    if ws is None:
        if write is not None or dwrite is not None:
            raise ValueError(f"{variant} takes no write gate")
    else:
        _need(write, "write", ws, torch.float32, dev)
        _need(dwrite, "dwrite", ws, torch.float32, dev)
    N = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    for t, name in ((S0, "S0"), (dS_T, "dS_T"), (dS0, "dS0")):
        if t is not None:
            _need(t, name, (N, H, dk_, dv_), torch.float32, dev)
    _need(dO, "dO", (B, T, H, dv_), torch.float32, dev)
    for t, name, shape in ((dq, "dq", (B, T, H, dk_)), (dk, "dk", (B, T, H) + nt + (dk_,)),
                           (dv, "dv", (B, T, H) + nt + (dv_,)), (dalpha, "dalpha", (B, T, H, dk_)),
                           (derase, "derase", es)):
        _need(t, name, shape, torch.float32, dev)
    if checkpoints is not None:
        # rows: sum over the sequences of floor(len / 64) (32 for product2); for packed sequences
        # that needs the lengths on the host, which a graph capture cannot read
        every = 32 if variant == "product2" else 64
        if cu_seqlens is None:
            rows = B * (T // every)
        elif not _capturing():
            rows = snapshot_count(check_offsets(cu_seqlens, T), every)
        else:
            rows = checkpoints.shape[0]
        _need(checkpoints, "checkpoints", (rows, H, dk_, dv_), torch.float32, dev)
    d = _dims_for(B, T, H, dk_, dv_, N, q.dtype, strides)
    with torch.cuda.device(dev):
        st = lib.dr_chunk_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write), VARIANTS[variant],
                                 _ptr(S0), _ptr(cu_seqlens), _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(dalpha), _ptr(derase), _ptr(dwrite), _ptr(dS0), _ptr(checkpoints),
                                 _dims_arg(d), _stream(dev))
    _check(lib, st, "dr_chunk_bwd")


def chunk_bwd(q, k, v, alpha, erase, write=None, variant: str = "kda", S0=None, cu_seqlens=None, dO=None,
              dS_T=None, need_dS0: bool = True, checkpoints=None):
    """Allocate the gradients and run ``dr_chunk_bwd``. Returns a dict with dq, dk, dv, dalpha,
    derase, dwrite (None for KDA / CKDA) and dS0 (None unless ``need_dS0``). ``checkpoints`` as
    for ``dr_chunk_bwd``."""
    f = lambda x: torch.empty(x.shape, dtype=torch.float32, device=q.device)
    N = q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1
    if cu_seqlens is not None and not _capturing():
        check_offsets(cu_seqlens, q.shape[1])
    g = dict(dq=f(q), dk=f(k), dv=f(v), dalpha=f(alpha), derase=f(erase),
             dwrite=None if write is None else f(write),
             dS0=torch.empty((N, q.shape[2], q.shape[3], v.shape[-1]), dtype=torch.float32, device=q.device)
             if need_dS0 else None)
    dr_chunk_bwd(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, dO, dS_T, g["dq"], g["dk"], g["dv"],
                 g["dalpha"], g["derase"], g["dwrite"], g["dS0"], checkpoints)
    return g


class _DeltaRule(torch.autograd.Function):
    """``chunk_fwd`` as an autograd node. The forward stores the states after every 64 tokens (32
    for product2) as the backward's checkpoints, so the backward runs only its reverse walk
    (``dr_chunk_bwd_ex``). Both directions are the library's kernels; this class only wires their
    tensors into torch's graph."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, erase, write, S0, cu_seqlens, variant, checkpoint):
        ctx.set_materialize_grads(False)  # an output that the loss does not use gets no gradient
        every = 32 if variant == "product2" else 64
        if checkpoint:
            o, S_T, ck = chunk_fwd(q, k, v, alpha, erase, write, variant, S0, cu_seqlens, snapshot_every=every)
        else:
            (o, S_T), ck = chunk_fwd(q, k, v, alpha, erase, write, variant, S0, cu_seqlens), None
        ctx.save_for_backward(q, k, v, alpha, erase, write, S0, cu_seqlens, ck)
        ctx.variant = variant
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, alpha, erase, write, S0, cu_seqlens, ck = ctx.saved_tensors
        if dO is None:
            dO = torch.zeros(q.shape[:3] + (v.shape[-1],), dtype=torch.float32, device=q.device)
        g = chunk_bwd(q, k, v, alpha, erase, write, ctx.variant, S0, cu_seqlens, dO=dO.contiguous(),
                      dS_T=None if dS_T is None else dS_T.contiguous(),
                      need_dS0=S0 is not None and ctx.needs_input_grad[6], checkpoints=ck)
        cast = lambda grad, x: None if grad is None else grad.to(x.dtype)
        return (cast(g["dq"], q), cast(g["dk"], k), cast(g["dv"], v), g["dalpha"], g["derase"], g["dwrite"],
                g["dS0"], None, None, None)


def delta_rule(q, k, v, alpha, erase, write=None, variant: str = "kda", S0=None, cu_seqlens=None,
               checkpoint: bool = True):
    """The prefill with gradients through torch autograd: returns (o, S_T) like ``chunk_fwd``;
    ``backward()`` on anything computed from them fills the ``.grad`` of q, k, v, alpha, erase,
    write and S0 (gradients of bf16 q, k, v are computed in fp32 and returned in bf16).
    ``checkpoint=False`` keeps no states from the forward (the backward then recomputes them,
    at about 5% of its time, with identical results)."""
    return _DeltaRule.apply(q, k, v, alpha, erase, write, S0, cu_seqlens, variant, checkpoint)
