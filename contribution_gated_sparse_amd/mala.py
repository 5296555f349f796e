"""Thin Python binding of libmala (ctypes). Argument marshalling only: every
step of the operator runs in the library's HIP kernels on the caller's current
stream. PyTorch is used for device memory and streams.

Functions carry the names of the C entry points: ``mala_fwd``, ``mala_bwd``,
``mala_decode``, ``mala_get_tiling``; the C ABI is documented in
``include/mala.h``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmala.so")

MALA_OK, MALA_ERR_INVALID_ARG, MALA_ERR_UNSUPPORTED, MALA_ERR_WORKSPACE, MALA_ERR_HIP = range(5)
MALA_F32, MALA_BF16 = 0, 1
OP_FWD, OP_BWD, OP_DECODE = 0, 1, 2


class MalaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmala status {status}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("n_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("tau", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("flags", ctypes.c_int32)]


MALA_FLAG_FAST_GRAD = 1
MALA_FLAG_GATE_PASS = 2


class DecodeProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cache_capacity", ctypes.c_int32), ("max_n_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("tau", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("split_keys", ctypes.c_int32)]


DECODE_SPLIT_AUTO = -1

EXPORTS = ("mala_get_tiling", "mala_fwd", "mala_bwd_workspace_size", "mala_bwd",
           "mala_bwd_nested", "mala_bwd_auto", "mala_bwd_stage", "mala_decode_workspace_size",
           "mala_decode_split_keys", "mala_decode", "mala_decode_stage", "mala_decode_noalloc",
           "mala_last_error", "mala_version")
BWD_PREP, BWD_DKDV, BWD_DQ = 0, 1, 2
DECODE_SPLIT, DECODE_COMBINE = 0, 1

_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmala.so (built in place by ``contribution_gated_sparse_amd.build``).
    Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmala.so not found at {p}; build it with "
                           "`python -m contribution_gated_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    P = ctypes.POINTER(Problem)
    DP = ctypes.POINTER(DecodeProblem)
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.mala_get_tiling.argtypes = [i32, i32, i32, pi32, pi32, pi32]
    lib.mala_get_tiling.restype = i32
    lib.mala_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mala_fwd.restype = i32
    lib.mala_bwd_workspace_size.argtypes = [P]
    lib.mala_bwd_workspace_size.restype = sz
    lib.mala_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_bwd.restype = i32
    lib.mala_bwd_nested.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_bwd_nested.restype = i32
    lib.mala_bwd_auto.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_bwd_auto.restype = i32
    lib.mala_bwd_stage.argtypes = [i32, P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_bwd_stage.restype = i32
    lib.mala_decode_stage.argtypes = [i32, DP, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_decode_stage.restype = i32
    lib.mala_decode_workspace_size.argtypes = [DP]
    lib.mala_decode_workspace_size.restype = sz
    lib.mala_decode_split_keys.argtypes = [DP]
    lib.mala_decode_split_keys.restype = i32
    lib.mala_decode.argtypes = [DP, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.mala_decode.restype = i32
    lib.mala_decode_noalloc.argtypes = [DP, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mala_decode_noalloc.restype = i32
    lib.mala_last_error.argtypes = []
    lib.mala_last_error.restype = ctypes.c_char_p
    lib.mala_version.argtypes = []
    lib.mala_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != MALA_OK:
        msg = load_library().mala_last_error().decode()
        raise MalaError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MALA_BF16
    if t.dtype == torch.float32:
        return MALA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mala_get_tiling(op: int, dtype: int = MALA_BF16, head_dim: int = 128):
    bq, bk, ch = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().mala_get_tiling(op, dtype, head_dim, ctypes.byref(bq),
                                          ctypes.byref(bk), ctypes.byref(ch)))
    return bq.value, bk.value, ch.value


def make_problem(q: torch.Tensor, k: torch.Tensor, tau: float, causal: bool = True,
                 softmax_scale: Optional[float] = None, flags: int = 0) -> Problem:
    b, hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    return Problem(b, hq, hkv, nq, nk, d, _dtype_code(q), 1 if causal else 0, float(tau),
                   float(scale), int(flags))


def mala_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float, causal: bool = True,
             softmax_scale: Optional[float] = None, want_mask: bool = False,
             want_kept: bool = True, out: Optional[dict] = None) -> dict:
    """Forward. q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> dict(o, lse, mask, kept)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    p = make_problem(q, k, tau, causal, softmax_scale)
    bq, bk, _ = mala_get_tiling(OP_FWD)
    tr, tc = -(-p.n_q // bq), -(-p.n_k // bk)
    if out is None:
        out = {}
    o = out.get("o")
    if o is None:
        o = torch.empty_like(q)
    lse = out.get("lse")
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    mask = out.get("mask") if want_mask else None
    if want_mask and mask is None:
        mask = torch.empty((p.batch, p.n_q_heads, tr, tc), dtype=torch.int8, device=q.device)
    kept = out.get("kept") if want_kept else None
    if want_kept and kept is None:
        kept = torch.empty((p.batch, p.n_q_heads, tr), dtype=torch.int32, device=q.device)
    _check(load_library().mala_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(mask), _ptr(kept), _stream()))
    return dict(o=o, lse=lse, mask=mask, kept=kept)


def mala_bwd(q, k, v, o, lse, d_o, tau: float, causal: bool = True,
             softmax_scale: Optional[float] = None, want_mask: bool = False,
             want_kept: bool = True, out: Optional[dict] = None, fast_grad: bool = False,
             gate_pass: bool = False, stages=None, events=None,
             fwd_mask: Optional[torch.Tensor] = None,
             fwd_kept: Optional[torch.Tensor] = None) -> dict:
    """Backward -> dict(dq, dk, dv, mask, kept). ``gate_pass``: take the
    decisions in a separate score pass so that dK/dV visits only the steps
    with a kept tile (MALA_FLAG_GATE_PASS). ``fwd_mask``: the forward's tile
    mask (``mala_fwd(..., want_mask=True)["mask"]``) for the same inputs; the
    score pass then forms only the scores of the tiles the forward kept
    (mala_bwd_nested, which runs in the gate-pass mode, so ``gate_pass`` is
    implied). ``fwd_kept``: the forward's kept-tile counters
    (``mala_fwd(...)["kept"]``) for the same inputs; the backward then
    chooses on the device between the gate-pass walks and the default walk,
    from its own decisions on a sample of the key tiles, or from the
    forward's counters when the sample is small (mala_bwd_auto; ``gate_pass``
    must be False). ``stages``: run only these
    stages (BWD_PREP, BWD_DKDV, BWD_DQ) through mala_bwd_stage; ``events``:
    optional list of torch.cuda.Event, one recorded after each stage run."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (d_o, "d_o")):
        _dev(t, n)
    if fwd_mask is not None:
        _dev(fwd_mask, "fwd_mask")
        if fwd_mask.dtype != torch.int8:
            raise TypeError("fwd_mask must be int8 (the forward's tile mask)")
        fb, fk, _ = mala_get_tiling(OP_FWD)
        want = (q.shape[0], q.shape[1], -(-q.shape[2] // fb), -(-k.shape[2] // fk))
        if tuple(fwd_mask.shape) != want:
            raise ValueError(f"fwd_mask has shape {tuple(fwd_mask.shape)}, expected {want}")
        if stages is not None or events is not None:
            raise ValueError("fwd_mask runs the whole backward: no stages or events")
        gate_pass = True
    if fwd_kept is not None:
        _dev(fwd_kept, "fwd_kept")
        if fwd_kept.dtype != torch.int32:
            raise TypeError("fwd_kept must be int32 (the forward's kept-tile counters)")
        fb, _, _ = mala_get_tiling(OP_FWD)
        want = (q.shape[0], q.shape[1], -(-q.shape[2] // fb))
        if tuple(fwd_kept.shape) != want:
            raise ValueError(f"fwd_kept has shape {tuple(fwd_kept.shape)}, expected {want}")
        if gate_pass or fwd_mask is not None or stages is not None or events is not None:
            raise ValueError("fwd_kept chooses the walk itself: no gate_pass, fwd_mask, stages or events")
    p = make_problem(q, k, tau, causal, softmax_scale,
                     (MALA_FLAG_FAST_GRAD if fast_grad else 0) | (MALA_FLAG_GATE_PASS if gate_pass else 0))
    lib = load_library()
    bq, bk, _ = mala_get_tiling(OP_BWD)
    tr, tc = -(-p.n_q // bq), -(-p.n_k // bk)
    out = {} if out is None else out
    dq = out.get("dq")
    dq = torch.empty_like(q) if dq is None else dq
    dk = out.get("dk")
    dk = torch.empty_like(k) if dk is None else dk
    dv = out.get("dv")
    dv = torch.empty_like(v) if dv is None else dv
    if fwd_kept is not None:    # the gate-pass workspace, whichever walk runs
        pg = make_problem(q, k, tau, causal, softmax_scale, p.flags | MALA_FLAG_GATE_PASS)
        nws = lib.mala_bwd_workspace_size(ctypes.byref(pg))
    else:
        nws = lib.mala_bwd_workspace_size(ctypes.byref(p))
    ws = out.get("ws")
    if ws is None or ws.numel() < nws:
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=q.device)
    mask = out.get("mask") if want_mask else None
    if want_mask and mask is None:
        mask = torch.empty((p.batch, p.n_q_heads, tr, tc), dtype=torch.int8, device=q.device)
    kept = out.get("kept") if want_kept else None
    if want_kept and kept is None:
        kept = torch.empty((p.batch, p.n_q_heads, tr), dtype=torch.int32, device=q.device)
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _ptr(mask), _ptr(kept), _stream())
    if fwd_mask is not None:
        _check(lib.mala_bwd_nested(*args[:7], _ptr(fwd_mask), *args[7:]))
    elif fwd_kept is not None:
        _check(lib.mala_bwd_auto(*args[:7], _ptr(fwd_kept), *args[7:]))
    elif stages is None and events is None:
        _check(lib.mala_bwd(*args))
    else:
        for n, stg in enumerate(stages if stages is not None else (BWD_PREP, BWD_DKDV, BWD_DQ)):
            _check(lib.mala_bwd_stage(stg, *args))
            if events is not None:
                events[n].record()
    return dict(dq=dq, dk=dk, dv=dv, mask=mask, kept=kept, ws=ws)


def make_decode_problem(q, k_cache, tau: float, max_n_k: int,
                        softmax_scale: Optional[float] = None,
                        split_keys: int = 0) -> DecodeProblem:
    b, hq, d = q.shape
    hkv, cap = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    return DecodeProblem(b, hq, hkv, d, cap, int(max_n_k), _dtype_code(q), float(tau), float(scale),
                         int(split_keys))


def decode_split_keys(p: DecodeProblem) -> int:
    """Keys per split that mala_decode uses for problem ``p`` (raises if
    ``p`` is invalid)."""
    lib = load_library()
    n = lib.mala_decode_split_keys(ctypes.byref(p))
    if n <= 0:
        raise MalaError(MALA_ERR_INVALID_ARG, lib.mala_last_error().decode())
    return n


def mala_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                seqlens_k: torch.Tensor, tau: float, max_n_k: Optional[int] = None,
                softmax_scale: Optional[float] = None, want_mask: bool = False,
                want_kept: bool = True, out: Optional[dict] = None, events=None,
                split_keys: int = 0, noalloc: bool = False) -> dict:
    """One split-KV decode step. q [B,Hq,d]; caches [B,Hkv,cap,d]; seqlens_k
    int32 [B] on the device (N_k including the current token). ``split_keys``:
    0 for the default split, DECODE_SPLIT_AUTO, or a multiple of 64; the
    returned ``split`` is the length used (the mask is [B,Hq,n_chunks,split/64]).
    ``noalloc``: call mala_decode_noalloc, which takes no workspace (the
    library's fixed device scratch; outputs are still allocated here unless
    given in ``out``)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seqlens_k, "seqlens_k")):
        _dev(t, n)
    if seqlens_k.dtype != torch.int32:
        raise TypeError("seqlens_k must be int32")
    if max_n_k is None:
        max_n_k = k_cache.shape[2]
    p = make_decode_problem(q, k_cache, tau, max_n_k, softmax_scale, split_keys)
    lib = load_library()
    _, bk, _ = mala_get_tiling(OP_DECODE)
    chunk = decode_split_keys(p)
    nch = -(-int(max_n_k) // chunk)
    out = {} if out is None else out
    o = out.get("o")
    o = torch.empty_like(q) if o is None else o
    lse = out.get("lse")
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    ws = None
    if not noalloc:
        nws = lib.mala_decode_workspace_size(ctypes.byref(p))
        ws = out.get("ws")
        if ws is None or ws.numel() < nws:
            ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=q.device)
    mask = out.get("mask") if want_mask else None
    if want_mask and mask is None:
        mask = torch.empty((p.batch, p.n_q_heads, nch, chunk // bk), dtype=torch.int8,
                           device=q.device)
    kept = out.get("kept") if want_kept else None
    if want_kept and kept is None:
        kept = torch.empty((p.batch, p.n_q_heads + p.n_kv_heads), dtype=torch.int32,
                           device=q.device)
    if noalloc:
        if events is not None:
            raise ValueError("noalloc runs the whole decode step: no events")
        _check(lib.mala_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(seqlens_k), _ptr(o), _ptr(lse), _ptr(mask),
                                       _ptr(kept), _stream()))
        return dict(o=o, lse=lse, mask=mask, kept=kept, ws=None, split=chunk)
    args = (ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o),
            _ptr(lse), _ptr(ws), ws.numel(), _ptr(mask), _ptr(kept), _stream())
    if events is None:
        _check(lib.mala_decode(*args))
    else:
        for n, stg in enumerate((DECODE_SPLIT, DECODE_COMBINE)):
            _check(lib.mala_decode_stage(stg, *args))
            events[n].record()
    return dict(o=o, lse=lse, mask=mask, kept=kept, ws=ws, split=chunk)


def version() -> str:
    return load_library().mala_version().decode()
