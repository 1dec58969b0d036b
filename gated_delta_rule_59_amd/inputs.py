"""Seeded synthetic inputs for the KDA workloads.

This module only draws random numbers and shapes them (normalise, squash,
round to the storage dtype). It holds none of the recurrence's arithmetic, so
both the HIP path and the CPU reference can consume what it makes.

Workloads (shapes and distributions of the Kimi K3 KDA layer; see the
"Eine Untergrenze, die einen GPU-Codepfad beseitigte" section of the orkas.ai
Kimi K3 architecture page for the -5 floor on the per-step log-decay):

  0  tiny-f32     B=1, H=2,  T=64,    dk=dv=32,  chunk 16, fp32 everything, S0 = 0
  1  prefill-4k   B=1, H=16, T=4096,  dk=dv=128, chunk 64, bf16 activations, S0 ~ 0.02 N(0,1)
  2  prefill-64k  B=1, H=32, T=65536, dk=dv=128, chunk 64, bf16, half of each head's key
                  channels pinned at g = -5 + 1e-3 (bf16 rounds that to -5.0 exactly)
  3  varlen-16    16 packed sequences, lengths uniform in [512, 16384], H=32, dk=dv=128, bf16
  4  decode-512   N=512 sequences, H=32, dk=dv=128, fp32 state 0.02 N(0,1) (1 GiB), bf16 token
                  inputs, a pool of 16 seeded step-input sets cycled over the steps
  5  unbounded-4k prefill-4k with g = -20 sigmoid(N(0,1)) (the decay-bound ablation's inputs)
  6  long memory  g = f sigmoid(N(0,1)) for a small |f| (test cases: the carried state dominates)

Every array is produced in float32 and then rounded to the storage dtype; the
float32 arrays returned hold exactly the values the kernels receive.
Seeding: tensor X of workload w is drawn in blocks of 1024 tokens (states: 64
(sequence, head) pairs), block i from numpy.random.default_rng([0, w, X, i]) with
X = 1 q, 2 k, 3 v, 4 beta, 5 g, 6 S0; the varlen lengths from default_rng([0, w, 0]) and the
pinned-channel mask from default_rng([0, w, 7]). Decode step-input set p uses the prefix
[0, 4, 1 + p]. Blocks are independent, so they are drawn on parallel threads.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GATE_FLOOR = -5.0          # per-step log-decay lower bound (retain >= e^-5 = 0.67 %)
DECODE_POOL = 16           # distinct seeded step-input sets for the decode workload


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


@dataclass
class Workload:
    name: str
    wid: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str                      # storage dtype of q, k, v, g, beta and o: "f32" | "bf16"
    B: int = 1
    T: int = 0                      # tokens per batch row (packed total when cu_seqlens is set)
    lengths: Optional[list] = None  # varlen sequence lengths
    n_seq: int = 1


@dataclass
class KDAInputs:
    """q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H]; S0: [n_seq, H, dk, dv] or None.

    cu_seqlens: int32 [n_seq + 1] token offsets into the packed T axis (B == 1), or None
    for a dense batch of B sequences of length T.
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    S0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


_TOK_BLOCK = 1024
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def _blocks(n, size):
    return [(a, min(a + size, n)) for a in range(0, n, size)]


def _draw(key, tensor, shape, transform, dtype, block=_TOK_BLOCK):
    """float32 array of `shape`; axis 0 is cut into blocks, block i drawn from
    default_rng([*key, tensor, i]) as N(0,1), then transform(), then rounded to dtype."""
    out = np.empty(shape, dtype=np.float32)

    def work(i_ab):
        i, (a, b) = i_ab
        rng = np.random.default_rng([*key, tensor, i])
        x = rng.standard_normal(size=(b - a,) + tuple(shape[1:]), dtype=np.float32)
        out[a:b] = to_storage(transform(x), dtype)

    list(_pool().map(work, enumerate(_blocks(shape[0], block))))
    return out


def _unit_rows(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))


def _sigmoid(x):
    return np.float32(1.0) / (np.float32(1.0) + np.exp(-x))


def draw_activations(key, B, T, H, dk, dv, dtype, gate_floor=GATE_FLOOR):
    """q, k unit rows over dk; v ~ N(0,1); beta = sigmoid(N(0,1)); g = gate_floor sigmoid(N(0,1))
    (gate_floor -5 everywhere except the unbounded-decay ablation inputs).
    Shapes [B, T, H, d] ([B, T, H] for beta); drawn over the flattened B*T token axis."""
    n = B * T
    q = _draw(key, 1, (n, H, dk), _unit_rows, dtype).reshape(B, T, H, dk)
    k = _draw(key, 2, (n, H, dk), _unit_rows, dtype).reshape(B, T, H, dk)
    v = _draw(key, 3, (n, H, dv), lambda x: x, dtype).reshape(B, T, H, dv)
    beta = _draw(key, 4, (n, H), _sigmoid, dtype).reshape(B, T, H)
    g = _draw(key, 5, (n, H, dk), lambda x: np.float32(gate_floor) * _sigmoid(x),
              dtype).reshape(B, T, H, dk)
    return q, k, v, g, beta


def draw_state(key, n, H, dk, dv, std=0.02):
    """fp32 states [n, H, dk, dv] ~ std * N(0,1), blocks of 64 (sequence, head) pairs."""
    x = _draw(key, 6, (n * H, dk, dv), lambda z: np.float32(std) * z, "f32", block=64)
    return x.reshape(n, H, dk, dv)


WORKLOADS = {
    0: Workload("tiny-f32", 0, H=2, dk=32, dv=32, chunk=16, dtype="f32", B=1, T=64),
    1: Workload("prefill-4k", 1, H=16, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=4096),
    2: Workload("prefill-64k-bound", 2, H=32, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=65536),
    3: Workload("varlen-16", 3, H=32, dk=128, dv=128, chunk=64, dtype="bf16", B=1, n_seq=16),
    4: Workload("decode-512", 4, H=32, dk=128, dv=128, chunk=0, dtype="bf16", B=512, T=1, n_seq=512),
}


def make_prefill(wid: int, *, T: Optional[int] = None, H: Optional[int] = None,
                 n_seq: Optional[int] = None) -> KDAInputs:
    """Inputs of prefill workload `wid` (0..3). T / H / n_seq override the sizes for
    reduced-size test cases (same distributions and structure, same seed)."""
    base = WORKLOADS[wid]
    wl = Workload(**{**base.__dict__})
    if H is not None:
        wl.H = H
    key = (0, wid)
    cu = None
    if wid == 3:
        ns = n_seq if n_seq is not None else base.n_seq
        lo, hi = (512, 16384) if T is None else (max(1, T // 4), T)
        rng = np.random.default_rng([*key, 0])
        lens = rng.integers(lo, hi, size=ns, endpoint=True).astype(np.int64)
        wl.lengths = [int(x) for x in lens]
        wl.n_seq = ns
        wl.T = int(lens.sum())
        cu = np.zeros(ns + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
    elif T is not None:
        wl.T = T
    q, k, v, g, beta = draw_activations(key, wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.dtype)
    S0 = None
    if wid != 0:
        S0 = draw_state(key, wl.n_seq if wid == 3 else wl.B, wl.H, wl.dk, wl.dv)
    extra = {}
    if wid == 2:
        rng = np.random.default_rng([*key, 7])
        pinned = np.zeros((wl.H, wl.dk), dtype=bool)
        for h in range(wl.H):
            pinned[h, rng.permutation(wl.dk)[: wl.dk // 2]] = True
        g[:, :, pinned] = to_storage(np.float32(GATE_FLOOR + 1e-3), wl.dtype)
        extra["pinned_channels"] = pinned
    return KDAInputs(wl, q, k, v, g, beta, S0, cu, extra)


def make_decode_state(N: int = 512, H: int = 32, dk: int = 128, dv: int = 128) -> np.ndarray:
    """Decode workload state: fp32 [N, H, dk, dv] ~ 0.02 N(0,1) (1 GiB at the full size)."""
    return draw_state((0, 4), N, H, dk, dv)


def make_decode_step(p: int, N: int = 512, H: int = 32, dk: int = 128, dv: int = 128):
    """Step-input set p of the decode workload: q, k, g [N, H, dk], v [N, H, dv], beta [N, H]
    in bf16 values, drawn as for prefill-4k. Step s of a run uses set s % DECODE_POOL."""
    q, k, v, g, beta = draw_activations((0, 4, 1 + p), N, 1, H, dk, dv, "bf16")
    return q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0]


UNBOUNDED_FLOOR = -20.0    # the ablation's per-step log-decay floor (the -5 bound removed)


def make_unbounded(T: int = 4096, H: int = 16, B: int = 1) -> KDAInputs:
    """prefill-4k's shapes and distributions with g = -20 sigmoid(N(0,1)): per-step decay down
    to e^-20, so a 16-token tile's cumulative log-decay reaches -320 and the dense diagonal-tile
    factorisation would need factors up to e^320 (the pairwise-diagonal ablation's inputs)."""
    key = (0, 5)
    q, k, v, g, beta = draw_activations(key, B, T, H, 128, 128, "bf16", gate_floor=UNBOUNDED_FLOOR)
    S0 = draw_state(key, B, H, 128, 128)
    wl = Workload("unbounded-4k", 5, H, 128, 128, 64, "bf16", B=B, T=T, n_seq=B)
    return KDAInputs(wl, q, k, v, g, beta, S0)


def make_long_memory(gate_floor: float, T: int = 2048, H: int = 2, B: int = 1) -> KDAInputs:
    """prefill-4k's distributions with a weak decay, g = gate_floor sigmoid(N(0,1)) for a small
    |gate_floor| (e.g. -0.1 or -0.01): the state keeps most of itself across a 64-token chunk
    (e^{-0.16} per chunk on average at -0.01), so what is carried from chunk to chunk, and
    from segment to segment, dominates the outputs. (At the recipe's -5 the state entering a
    chunk has decayed by about e^-160 before the chunk ends.)"""
    key = (0, 6, int(round(-gate_floor * 1e4)))
    q, k, v, g, beta = draw_activations(key, B, T, H, 128, 128, "bf16", gate_floor=gate_floor)
    S0 = draw_state(key, B, H, 128, 128)
    wl = Workload(f"long-memory g>={gate_floor}", 6, H, 128, 128, 64, "bf16", B=B, T=T, n_seq=B)
    return KDAInputs(wl, q, k, v, g, beta, S0)
