"""The chunked algebra (tests/chunked_model.py) equals the sequential oracle in float64,
including at the decay floor, for every chunk length the kernels take; and the
per-16-token-tile reference is what keeps the factored products finite."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.chunked_model import chunk_matrices, chunked_forward


def rel(a, b):
    return np.abs(a - b).max() / np.sqrt(np.mean(np.square(b)))


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_equals_oracle(chunk):
    x = inputs.make_prefill(1, T=300, H=2)
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
    o, s = chunked_forward(x.q, x.k, x.v, x.g, x.beta, x.S0, chunk=chunk)
    assert rel(o, o_ref) < 1e-12 and rel(s, s_ref) < 1e-12


def test_chunked_equals_oracle_at_decay_floor_and_varlen():
    x = inputs.make_prefill(2, T=512, H=2)
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
    o, s = chunked_forward(x.q, x.k, x.v, x.g, x.beta, x.S0, chunk=64)
    assert rel(o, o_ref) < 1e-12 and rel(s, s_ref) < 1e-12
    y = inputs.make_prefill(3, T=200, H=2, n_seq=4)
    o_ref, s_ref = oracle.kda_reference(y.q, y.k, y.v, y.g, y.beta, y.S0, cu_seqlens=y.cu_seqlens)
    o, s = chunked_forward(y.q, y.k, y.v, y.g, y.beta, y.S0, cu_seqlens=y.cu_seqlens, chunk=64)
    assert rel(o, o_ref) < 1e-12 and rel(s, s_ref) < 1e-12


def test_tile_reference_keeps_factors_finite_in_fp32():
    """All g at the floor (-5): within a 64-token chunk G reaches -320. Factoring from the
    tile start keeps every factor of the products inside fp32 (and bf16) range; factoring
    from the chunk start overflows (e^320 = inf) and poisons the products."""
    rng = np.random.default_rng(0)
    C, dk = 64, 16
    k = rng.standard_normal((C, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((C, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    g = np.full((C, dk), -5.0)
    Akk, Aqk, G = chunk_matrices(q, k, g, factor_dtype=np.float32)
    assert np.isfinite(Akk).all() and np.isfinite(Aqk).all()
    exact = np.tril(np.einsum("rc,jc,rjc->rj", k, k, np.exp(G[:, None, :] - G[None, :, :])))
    np.testing.assert_allclose(Akk, exact, rtol=1e-5, atol=1e-30)
    bad, _, _ = chunk_matrices(q, k, g, factor_dtype=np.float32, single_reference=True)
    assert not np.isfinite(bad).all()
    # within one tile the worst column factor is e^80: finite in bf16 and fp32
    assert np.float32(np.exp(80.0)) < inputs.round_to_bf16(np.array([3.0e38], np.float32))[0]
