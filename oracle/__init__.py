"""CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may import this package. The library (``gated_delta_rule_59_amd``)
never imports it, and it imports nothing from the library.

What it computes (one (sequence, head) chain at a time, token by token, state S of
size dk x dv with rows indexed by key channel)::

    S <- Diag(exp(g_t)) S          decay of the incoming state
    u <- v_t - S^T k_t             what the decayed state mispredicts for k_t
    S <- S + beta_t k_t u^T        delta-rule write
    o_t <- S^T q_t                 read after the update

Sources: the fixed-size decaying running state is described in the "Sequenz" section
of the orkas.ai Kimi K3 architecture page; the token-dependent transition applied to
the incoming state in its "Die Rechnung landet in der Bereitstellungsinfrastruktur"
section; the studioglobal.ai pages ("KDA haandterer ..." / "Architektur fuer lange
Kontexte ...") add that the state and the per-token decode work do not grow with the
context. The pages describe but never write out the update; the form above is the plain
gated delta-rule reading (decay before the erase, beta scales erase and write, output
read after the update, no scale on q).

The arithmetic lives in ``kda_oracle.c`` (plain C, OpenMP over independent chains).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/libkda_oracle.so."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    for name, real in (("kda_oracle_f64", ctypes.c_double), ("kda_oracle_f32", ctypes.c_float)):
        fn = getattr(lib, name)
        P = ctypes.c_void_p
        fn.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                       P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_reference(q, k, v, g, beta, S0=None, cu_seqlens=None, *, erase: bool = True,
                  precision: str = "f64", chains: Optional[Sequence[Sequence[int]]] = None,
                  threads: int = 0, want_state: bool = True):
    """Run the recurrence.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H] (any float dtype; converted
    to float32, which is exact for bf16 and fp32 data).
    S0: [n_seq, H, dk, dv] or None (zeros). n_seq = B, or len(cu_seqlens) - 1 when
    cu_seqlens (token offsets into the packed T axis, B must be 1) is given.
    chains: optional list of (sequence, head) pairs; only those are computed, the other
    rows of o (and S_T) are NaN.
    Returns (o [B, T, H, dv], S_T [n_seq, H, dk, dv] or None) in float64 (precision "f64")
    or float32 ("f32").
    """
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] or \
            beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch")
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        starts = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if starts[0] != 0 or starts[-1] != T or np.any(np.diff(starts) < 0):
            raise ValueError("bad cu_seqlens")
    else:
        starts = np.arange(B + 1, dtype=np.int64) * T
    n_seq = len(starts) - 1
    real = np.float64 if precision == "f64" else np.float32
    fn = lib.kda_oracle_f64 if precision == "f64" else lib.kda_oracle_f32
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=real)
        if s0.shape != (n_seq, H, dk, dv):
            raise ValueError(f"S0 shape {s0.shape} != {(n_seq, H, dk, dv)}")
    o = np.full((B, T, H, dv), np.nan, dtype=real)
    s_t = np.full((n_seq, H, dk, dv), np.nan, dtype=real) if want_state else None
    ch = None
    n_ch = 0
    if chains is not None:
        ch = np.ascontiguousarray(np.asarray(chains, dtype=np.int32).reshape(-1, 2))
        n_ch = ch.shape[0]
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(starts), n_seq, H, dk,
            dv, _ptr(ch), n_ch, 1 if erase else 0, _ptr(o), _ptr(s_t), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle failed with code {rc}")
    return o, s_t


def kda_decode_reference(q, k, v, g, beta, S, *, precision: str = "f64", chains=None,
                         threads: int = 0):
    """One decode step for N independent sequences: q, k, g [N, H, dk], v [N, H, dv],
    beta [N, H], S [N, H, dk, dv]. Returns (o [N, H, dv], S_new [N, H, dk, dv]).

    A decode step is the recurrence over a single token per sequence, so this is
    ``kda_reference`` with N sequences of length one."""
    N, H, dk = np.shape(q)
    o, s_new = kda_reference(np.reshape(q, (1, N, H, dk)), np.reshape(k, (1, N, H, dk)),
                             np.reshape(v, (1, N, H, -1)), np.reshape(g, (1, N, H, dk)),
                             np.reshape(beta, (1, N, H)), S,
                             cu_seqlens=np.arange(N + 1), precision=precision, chains=chains,
                             threads=threads)
    return o[0], s_new


def threads_used(threads: int = 0) -> int:
    """How many OpenMP threads a call with `threads` (0 = default) uses."""
    return int(threads) if threads > 0 else int(os.environ.get("OMP_NUM_THREADS", 0)) or \
        (os.cpu_count() or 1)
