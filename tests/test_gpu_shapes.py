"""Shapes and batch structures through the C ABI against the oracle: many packed sequences
(more than the walk orders by length, so the given order is kept), equal lengths (ties in
the longest-first order), and a seeded sweep of random dense and packed batches on both
prefill paths and on every head-dim pair of the fp32 path."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, host, kda_inputs_dev

pytestmark = pytest.mark.gpu


def packed(lengths, H, key, dtype="bf16", dk=128, dv=128):
    T = int(sum(lengths))
    q, k, v, g, beta = inputs.draw_activations(key, 1, T, H, dk, dv, dtype)
    S0 = inputs.draw_state(key, len(lengths), H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    wl = inputs.Workload("packed", 3, H, dk, dv, 64, dtype, B=1, T=T, lengths=list(lengths),
                         n_seq=len(lengths))
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0, cu)


def dense(B, T, H, key, dtype="bf16", dk=128, dv=128):
    q, k, v, g, beta = inputs.draw_activations(key, B, T, H, dk, dv, dtype)
    S0 = inputs.draw_state(key, B, H, dk, dv)
    wl = inputs.Workload("dense", 1, H, dk, dv, 64, dtype, B=B, T=T, n_seq=B)
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0)


def check(x, *, generic=False, chunk=64, tau=TAU["bf16"], label=""):
    import torch
    from gated_delta_rule_59_amd import binding
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    o, s = binding.chunk_fwd(q, k, v, g, beta, S0, cu, chunk=chunk, generic=generic)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens)
    assert_parity(host(o), o_ref, tau, f"{label} o")
    assert_parity(host(s), s_ref, tau, f"{label} S_T")


def test_many_packed_sequences():
    """600 packed sequences of 0..40 tokens (more than the walk ranks by length)."""
    lens = np.random.default_rng([0, 8, 1]).integers(0, 41, 600)
    print(f"600 sequences, {lens.sum()} tokens", flush=True)
    check(packed(lens, 2, (9, 81)), label="600 sequences")


def test_equal_length_sequences():
    """Ties in the longest-first order: 20 sequences of 100 tokens and 3 of 300."""
    lens = [100] * 10 + [300] + [100] * 10 + [300, 300]
    check(packed(lens, 3, (9, 82)), label="equal lengths")


def _random_cases(n=6):
    rng = np.random.default_rng([0, 8, 2])
    for i in range(n):
        H = int(rng.integers(1, 5))
        if i % 2:
            lens = [int(x) for x in rng.integers(0, 400, int(rng.integers(1, 9)))]
            yield f"packed {list(lens)} H={H}", lambda lens=lens, H=H, i=i: packed(lens, H, (9, 83, i))
        else:
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, 500))
            yield f"dense B={B} T={T} H={H}", lambda B=B, T=T, H=H, i=i: dense(B, T, H, (9, 83, i))


RANDOM = dict(_random_cases())


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
@pytest.mark.parametrize("name", list(RANDOM))
def test_random_shapes(name, generic):
    print(f"{name} generic={generic}", flush=True)
    check(RANDOM[name](), generic=generic, label=name)


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_fp32_path_every_head_dim_pair(dk, dv):
    """The fp32 path on every (dk, dv) it accepts, packed with ragged lengths, chunk 32."""
    check(packed([5, 70, 0, 33], 2, (9, 84, dk, dv), dtype="f32", dk=dk, dv=dv),
          generic=True, chunk=32, tau=TAU["f32"], label=f"fp32 dk={dk} dv={dv}")
