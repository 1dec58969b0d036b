"""Python binding of libkda (include/kda.h): torch tensors in, device pointers and the
current HIP stream out to the C ABI. Argument marshalling only; every step of the
computation runs in the library's kernels. Raises if the built library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_FLAG_GENERIC = 1
KDA_FLAG_PAIRWISE_DIAG = 2
KDA_FLAG_WALK64 = 4
KDA_FLAG_WALK128 = 8
ABI_VERSION = 4  # KDA_ABI_VERSION of include/kda.h this binding marshals for
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL_PTR", 2: "KDA_ERR_BAD_SHAPE", 3: "KDA_ERR_BAD_DTYPE",
          4: "KDA_ERR_UNSUPPORTED", 5: "KDA_ERR_DECAY_RANGE", 6: "KDA_ERR_WORKSPACE",
          7: "KDA_ERR_HIP", 8: "KDA_ERR_ALIAS"}

_P = ctypes.c_void_p
SIZE_MAX = ctypes.c_size_t(-1).value
CHECK_COUNTERS = 1024  # KDA_CHECK_COUNTERS
NOALLOC_SCRATCH_BYTES = 128 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class ChunkArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("chunk", ctypes.c_int),
                ("cu_seqlens", _P), ("N", ctypes.c_int),
                ("act_dtype", ctypes.c_int), ("gate_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
                ("S0", _P), ("o", _P), ("S_T", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint),
                ("ckpt", _P), ("ckpt_every", ctypes.c_int), ("ckpt_slots", ctypes.c_int),
                ("segments", ctypes.c_int)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int),
                ("act_dtype", ctypes.c_int), ("gate_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
                ("S", _P), ("o", _P)]


class DecodeMultiArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("m", ctypes.c_int),
                ("act_dtype", ctypes.c_int), ("gate_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
                ("S", _P), ("o", _P), ("accept", _P)]


class KDAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkda; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkda is not built ({LIB_PATH} missing); run "
                               "python -m gated_delta_rule_59_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkArgs)]
        L.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkArgs), _P]
        L.kda_chunk_fwd.restype = ctypes.c_int
        L.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkArgs), _P]
        L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        L.kda_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _P]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_decode_multi.argtypes = [ctypes.POINTER(DecodeMultiArgs), _P]
        L.kda_decode_multi.restype = ctypes.c_int
        L.kda_check_gates.argtypes = [_P, ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int, _P,
                                      ctypes.c_int, _P, ctypes.POINTER(ctypes.c_int64)]
        L.kda_check_gates.restype = ctypes.c_int
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.argtypes = []
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_abi_version.argtypes = []
        L.kda_abi_version.restype = ctypes.c_int
        if L.kda_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libkda ABI {L.kda_abi_version()} does not match the binding's "
                               f"{ABI_VERSION}; rebuild with python -m gated_delta_rule_59_amd.build")
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise KDAError(status, lib().kda_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _P(t.data_ptr())


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream) -> _P:
    s = torch.cuda.current_stream() if stream is None else stream
    return _P(s.cuda_stream)


def chunk_args(q, k, v, g, beta, S0=None, cu_seqlens=None, *, chunk=64, o=None, S_T=None,
               workspace=None, generic=False, ckpt=None, ckpt_every=0,
               pairwise_diag=False, segments=0, walk64=False, walk128=False) -> ChunkArgs:
    B, T, H, dk = q.shape
    a = ChunkArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = B, T, H, dk, v.shape[-1], chunk
    a.cu_seqlens = _ptr(cu_seqlens)
    a.N = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    a.act_dtype = _dtype_code(q.dtype)
    a.gate_dtype = _dtype_code(g.dtype)
    a.out_dtype = _dtype_code(o.dtype) if o is not None else KDA_F32
    a.q, a.k, a.v, a.g, a.beta = (_ptr(t) for t in (q, k, v, g, beta))
    a.S0, a.o, a.S_T = _ptr(S0), _ptr(o), _ptr(S_T)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.flags = ((KDA_FLAG_GENERIC if generic else 0) | (KDA_FLAG_PAIRWISE_DIAG if pairwise_diag else 0)
               | (KDA_FLAG_WALK64 if walk64 else 0) | (KDA_FLAG_WALK128 if walk128 else 0))
    a.ckpt = _ptr(ckpt)
    a.ckpt_every = ckpt_every
    a.ckpt_slots = 0 if ckpt is None else ckpt.shape[0]
    a.segments = segments
    return a


def checkpoint_slots(lengths, every: int) -> int:
    """Slots a checkpoint buffer needs for sequences of these lengths: one per full `every`
    tokens of each sequence (host-side arithmetic, the layout of kda_chunk_args.ckpt)."""
    return int(sum(int(n) // every for n in lengths)) if every > 0 else 0


def chunk_fwd_workspace_bytes(q, k, v, g, beta, S0=None, cu_seqlens=None, *, chunk=64,
                              generic=False, segments=0, walk64=False, walk128=False,
                              ckpt_every=0) -> int:
    a = chunk_args(q, k, v, g, beta, S0, cu_seqlens, chunk=chunk, generic=generic,
                   segments=segments, walk64=walk64, walk128=walk128, ckpt_every=ckpt_every)
    n = lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
    if n == SIZE_MAX:
        raise KDAError(2, lib().kda_last_error().decode())
    return int(n)


def alloc_workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Device scratch for kda_chunk_fwd (torch's allocator returns 256-byte aligned blocks)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, *, chunk=64,
              out_dtype=torch.float32, o=None, S_T=None, want_state=True, workspace=None,
              generic=False, stream=None, ckpt=None, ckpt_every=0, pairwise_diag=False,
              segments=0, walk64=False, walk128=False):
    """Prefill. q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H] (bf16 or fp32, on the
    GPU, contiguous); S0 [n_seq, H, dk, dv] fp32 or None; cu_seqlens int32 [N + 1] or None.
    Returns (o [B, T, H, dv] out_dtype, S_T [n_seq, H, dk, dv] fp32 or None).
    S_T may be passed as S0 itself to continue in place.
    ckpt_every > 0 (a multiple of chunk) also stores the state after every ckpt_every tokens
    of each sequence into ckpt [slots, H, dk, dv] fp32 (see checkpoint_slots).
    pairwise_diag evaluates the diagonal tiles pairwise (no lower bound on g needed; slower).
    segments (3 .. 8) walks each sequence in that many segments in parallel (see kda.h).
    walk64 / walk128 make the matrix-core walk take one 64-token chunk per step, or two
    chunks composed into one 128-token step (see kda.h; by default the library chooses)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev(t, name)
    if S0 is not None:
        _dev(S0, "S0")
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    else:
        _dev(o, "o")
    if S_T is None and want_state:
        S_T = torch.empty((n_seq, H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = chunk_fwd_workspace_bytes(q, k, v, g, beta, S0, cu_seqlens, chunk=chunk,
                                           generic=generic, segments=segments, walk64=walk64,
                                           walk128=walk128, ckpt_every=ckpt_every)
        workspace = alloc_workspace(nbytes, q.device)
    if ckpt_every:
        if ckpt is None:
            raise ValueError("ckpt_every needs a ckpt buffer (size it with checkpoint_slots)")
        _dev(ckpt, "ckpt")
        if ckpt.dtype != torch.float32 or tuple(ckpt.shape[1:]) != (H, dk, dv):
            raise ValueError("ckpt must be fp32 [slots, H, dk, dv]")
    a = chunk_args(q, k, v, g, beta, S0, cu_seqlens, chunk=chunk, o=o, S_T=S_T,
                   workspace=workspace, generic=generic, ckpt=ckpt if ckpt_every else None,
                   ckpt_every=ckpt_every, pairwise_diag=pairwise_diag, segments=segments,
                   walk64=walk64, walk128=walk128)
    _check(lib().kda_chunk_fwd(ctypes.byref(a), _stream(stream)))
    return o, S_T


def chunk_fwd_noalloc(q, k, v, g, beta, S0=None, cu_seqlens=None, *, o, S_T=None, chunk=64,
                      generic=False, stream=None, ckpt=None, ckpt_every=0, segments=0,
                      walk64=False, walk128=False):
    """kda_chunk_fwd_noalloc: the prefill with the library's fixed device scratch in place of
    a workspace; o (and S_T, ckpt when wanted) are the caller's, nothing is allocated here.
    Raises KDAError (KDA_ERR_WORKSPACE) when the sizes need more than NOALLOC_SCRATCH_BYTES."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o)):
        _dev(t, name)
    for name, t in (("S0", S0), ("S_T", S_T), ("cu_seqlens", cu_seqlens), ("ckpt", ckpt)):
        if t is not None:
            _dev(t, name)
    a = chunk_args(q, k, v, g, beta, S0, cu_seqlens, chunk=chunk, o=o, S_T=S_T,
                   generic=generic, ckpt=ckpt if ckpt_every else None, ckpt_every=ckpt_every,
                   segments=segments, walk64=walk64, walk128=walk128)
    _check(lib().kda_chunk_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return o, S_T


def decode_args(q, k, v, g, beta, S, o) -> DecodeArgs:
    N, H, dk = q.shape
    a = DecodeArgs()
    a.N, a.H, a.dk, a.dv = N, H, dk, v.shape[-1]
    a.act_dtype = _dtype_code(q.dtype)
    a.gate_dtype = _dtype_code(g.dtype)
    a.out_dtype = _dtype_code(o.dtype)
    a.q, a.k, a.v, a.g, a.beta, a.S, a.o = (_ptr(t) for t in (q, k, v, g, beta, S, o))
    return a


def decode_step(q, k, v, g, beta, S, *, o=None, out_dtype=torch.float32, stream=None):
    """One token per sequence: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H]; S [N, H, dk, dv]
    fp32 updated in place. Returns o [N, H, dv]."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S", S)):
        _dev(t, name)
    if o is None:
        o = torch.empty((q.shape[0], q.shape[1], v.shape[-1]), dtype=out_dtype, device=q.device)
    a = decode_args(q, k, v, g, beta, S, o)
    _check(lib().kda_decode_step(ctypes.byref(a), _stream(stream)))
    return o


def decode_multi(q, k, v, g, beta, S, *, accept=None, o=None, want_output=True,
                 out_dtype=torch.float32, stream=None):
    """m tokens per sequence from one read of S: q, k, g [N, m, H, dk]; v [N, m, H, dv];
    beta [N, m, H]; S [N, H, dk, dv] fp32. accept None: S unchanged (verification);
    accept int32 [N] on the GPU: S[n] <- state after its first accept[n] tokens (commit).
    Returns o [N, m, H, dv] (None when want_output is False and o is not given)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S", S)):
        _dev(t, name)
    N, m, H, dk = q.shape
    if accept is not None:
        _dev(accept, "accept")
        if accept.dtype != torch.int32 or accept.numel() != N:
            raise ValueError("accept must be int32 [N]")
    if o is None and want_output:
        o = torch.empty((N, m, H, v.shape[-1]), dtype=out_dtype, device=q.device)
    elif o is not None:
        _dev(o, "o")
    a = DecodeMultiArgs()
    a.N, a.H, a.dk, a.dv, a.m = N, H, dk, v.shape[-1], m
    a.act_dtype = _dtype_code(q.dtype)
    a.gate_dtype = _dtype_code(g.dtype)
    a.out_dtype = _dtype_code(o.dtype) if o is not None else KDA_F32
    a.q, a.k, a.v, a.g, a.beta, a.S = (_ptr(t) for t in (q, k, v, g, beta, S))
    a.o, a.accept = _ptr(o), _ptr(accept)
    _check(lib().kda_decode_multi(ctypes.byref(a), _stream(stream)))
    return o


def check_gates(g, beta, stream=None, counts=None) -> int:
    """Number of g values outside [-5, 0] plus beta values outside [0, 1] (synchronises).
    counts: int64 device scratch for the per-workgroup counters (allocated here if None)."""
    _dev(g, "g")
    _dev(beta, "beta")
    if counts is None:
        counts = torch.empty(CHECK_COUNTERS, dtype=torch.int64, device=g.device)
    _dev(counts, "counts")
    if counts.dtype != torch.int64:
        raise TypeError("counts must be int64")
    n = ctypes.c_int64(0)
    _check(lib().kda_check_gates(_ptr(g), g.numel(), _ptr(beta), beta.numel(),
                                 _dtype_code(g.dtype), _ptr(counts), counts.numel(),
                                 _stream(stream), ctypes.byref(n)))
    return int(n.value)
