"""Pins for the CPU oracle (oracle/): each test checks it against something other than
itself - a hand-worked example, a closed form, a library routine, an invariant of the
update, brute force with explicit transition matrices, or the numbers the pages print.
Chosen so that a dropped term, a flipped sign, a swapped order (decay vs erase, read
before vs after the write) or a transposed operand in the oracle fails at least one.
CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, T=10, H=2, dk=4, dv=3, unit=True, s0=True, B=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dk))))
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    f = lambda a: None if a is None else np.asarray(a, np.float32)  # noqa: E731
    return f(q), f(k), f(v), f(g), f(beta), (None if S0 is None else S0)


def rms(x):
    return float(np.sqrt(np.mean(np.square(x))))


# ---------------------------------------------------------------- P1 worked examples
def test_worked_example_scalar():
    """dk = dv = 1, g = ln(1/2), k = q = 1, beta = 1/2, v = (4, 2), S0 = 0, by hand:
    t=1: S = 0.5*0 = 0; u = 4 - 0 = 4; S = 0 + 0.5*4 = 2; o = 2.
    t=2: S = 0.5*2 = 1; u = 2 - 1 = 1; S = 1 + 0.5*1 = 1.5; o = 1.5."""
    one = np.ones((1, 2, 1, 1), np.float32)
    g = np.full((1, 2, 1, 1), math.log(0.5), np.float32)
    v = np.array([4.0, 2.0], np.float32).reshape(1, 2, 1, 1)
    beta = np.full((1, 2, 1), 0.5, np.float32)
    o, s = oracle.kda_reference(one, one, v, g, beta)
    np.testing.assert_allclose(o.ravel(), [2.0, 1.5], rtol=1e-7)
    np.testing.assert_allclose(s.ravel(), [1.5], rtol=1e-7)


def test_worked_example_2x2():
    """dk = dv = 2, one token, S0 = I, g = (0, ln 1/2), k = (0.6, 0.8), q = (1, 0),
    v = (1, -1), beta = 1. By hand: Diag(e^g) S0 = [[1, 0], [0, 0.5]];
    (Diag S0)^T k = (0.6, 0.4); u = v - that = (0.4, -1.4);
    S = [[1 + 0.24, -0.84], [0.32, 0.5 - 1.12]] = [[1.24, -0.84], [0.32, -0.62]];
    o = S^T q = (1.24, -0.84)."""
    f = lambda a, shp: np.array(a, np.float32).reshape(shp)  # noqa: E731
    q = f([1.0, 0.0], (1, 1, 1, 2))
    k = f([0.6, 0.8], (1, 1, 1, 2))
    v = f([1.0, -1.0], (1, 1, 1, 2))
    g = f([0.0, math.log(0.5)], (1, 1, 1, 2))
    beta = f([1.0], (1, 1, 1))
    S0 = np.eye(2).reshape(1, 1, 2, 2)
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o.ravel(), [1.24, -0.84], atol=1e-7)
    np.testing.assert_allclose(s.reshape(2, 2), [[1.24, -0.84], [0.32, -0.62]], atol=1e-7)


# ---------------------------------------------------------------- P2 brute force, unrolled
def test_bruteforce_unrolled_transitions():
    """S_t = Phi_t ... Phi_1 S0 + sum_s Phi_t ... Phi_{s+1} beta_s k_s v_s^T with the
    explicit dk x dk transitions Phi_t = (I - beta_t k_t k_t^T) Diag(exp g_t); o_t = S_t^T q_t."""
    q, k, v, g, beta, S0 = rand_case(1, T=9, H=2, dk=4, dv=3)
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    T, H, dk, dv = q.shape[1], q.shape[2], q.shape[3], v.shape[3]
    d = lambda a: np.asarray(a, np.float64)  # noqa: E731
    for h in range(H):
        phis, writes = [], []
        for t in range(T):
            kt = d(k[0, t, h])[:, None]
            phis.append((np.eye(dk) - beta[0, t, h] * kt @ kt.T) @ np.diag(np.exp(d(g[0, t, h]))))
            writes.append(beta[0, t, h] * kt @ d(v[0, t, h])[None, :])
        for t in range(T):
            def prod(a, b):  # Phi_b ... Phi_a (a <= b), identity when a > b
                m = np.eye(dk)
                for j in range(a, b + 1):
                    m = phis[j] @ m
                return m
            St = prod(0, t) @ S0[0, h]
            for s_ in range(t + 1):
                St = St + prod(s_ + 1, t) @ writes[s_]
            np.testing.assert_allclose(o[0, t, h], St.T @ d(q[0, t, h]), rtol=1e-12, atol=1e-12)
            if t == T - 1:
                np.testing.assert_allclose(s[0, h], St, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P3 literal beta = 0
def test_beta_zero_closed_form():
    """beta = 0 writes nothing: S_T = Diag(exp(sum g)) S0, o_t = (Diag(exp G_t) S0)^T q_t.
    A reading where beta only scales the erase (and the write is unscaled) fails this."""
    q, k, v, g, beta, S0 = rand_case(2, T=7)
    beta[:] = 0
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    G = np.cumsum(g.astype(np.float64), axis=1)
    for h in range(q.shape[2]):
        for t in range(q.shape[1]):
            np.testing.assert_allclose(o[0, t, h], (np.exp(G[0, t, h])[:, None] * S0[0, h]).T @
                                       q[0, t, h], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(s[0, h], np.exp(G[0, -1, h])[:, None] * S0[0, h], rtol=1e-12)
    g[:] = 0
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    np.testing.assert_allclose(s, S0, rtol=0, atol=0)
    np.testing.assert_allclose(o[0], np.einsum("thc,hcj->thj", q[0].astype(np.float64), S0[0]),
                               rtol=1e-12)


# ---------------------------------------------------------------- P4 gated linear attention
def gla_direct(q, k, v, g, beta, S0):
    """o_t = sum_{s<=t} beta_s ((q_t * exp(G_t - G_s)) . k_s) v_s + (Diag(exp G_t) S0)^T q_t,
    the O(T^2) form of gated linear attention (one batch row)."""
    q, k, v, g, beta = (np.asarray(a, np.float64)[0] for a in (q, k, v, g, beta))
    T, H, _ = q.shape
    G = np.cumsum(g, axis=0)
    o = np.zeros((T, H, v.shape[-1]))
    for h in range(H):
        for t in range(T):
            acc = np.zeros(v.shape[-1])
            for s_ in range(t + 1):
                acc += beta[s_, h] * np.dot(q[t, h] * np.exp(G[t, h] - G[s_, h]), k[s_, h]) * v[s_, h]
            if S0 is not None:
                acc += (np.exp(G[t, h])[:, None] * S0[0, h]).T @ q[t, h]
            o[t, h] = acc
    return o


def test_no_erase_is_gated_linear_attention():
    q, k, v, g, beta, S0 = rand_case(3, T=11)
    o, _ = oracle.kda_reference(q, k, v, g, beta, S0, erase=False)
    np.testing.assert_allclose(o[0], gla_direct(q, k, v, g, beta, S0), rtol=1e-11, atol=1e-12)


def test_small_beta_limit_is_gated_linear_attention():
    """KDA with beta = eps * b and S0 = 0 is, to first order in eps, gated linear attention
    with write weights b: d o / d eps at 0 = GLA(b). Richardson: 2 D(eps/2) - D(eps)."""
    q, k, v, g, b, _ = rand_case(4, T=10, s0=False)
    eps = 2.0 ** -12
    D = lambda e: oracle.kda_reference(q, k, v, g, (b * np.float32(e)).astype(np.float32))[0] / e  # noqa: E731
    rich = 2 * D(eps / 2) - D(eps)
    ref = gla_direct(q, k, v, g, b, None)
    assert np.abs(rich[0] - ref).max() <= 1e-6 * np.abs(ref).max()
    # and the first-order term is not the full KDA output at beta = b
    full = oracle.kda_reference(q, k, v, g, b)[0]
    assert np.abs(full[0] - ref).max() > 1e-2 * np.abs(ref).max()


# ---------------------------------------------------------------- P5 causal linear attention
def test_no_decay_no_erase_is_causal_linear_attention():
    """g = 0 and no erase: o = tril(Q K^T) (b * V) + Q S0, a library matmul. The inclusive
    diagonal (read after the write) is what makes tril include the diagonal."""
    q, k, v, g, b, S0 = rand_case(5, T=12, H=2, dk=5, dv=4)
    g[:] = 0
    o, _ = oracle.kda_reference(q, k, v, g, b, S0, erase=False)
    for h in range(q.shape[2]):
        Q, K, V = (np.asarray(a[0, :, h], np.float64) for a in (q, k, v))
        ref = np.tril(Q @ K.T) @ (b[0, :, h, None].astype(np.float64) * V) + Q @ S0[0, h]
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-12, atol=1e-12)
    # the beta -> 0 limit of the full recurrence gives the same (with S0 = 0)
    eps = 2.0 ** -12
    D = lambda e: oracle.kda_reference(q, k, v, g, (b * np.float32(e)).astype(np.float32))[0] / e  # noqa: E731
    rich = 2 * D(eps / 2) - D(eps)
    for h in range(q.shape[2]):
        Q, K, V = (np.asarray(a[0, :, h], np.float64) for a in (q, k, v))
        ref = np.tril(Q @ K.T) @ (b[0, :, h, None].astype(np.float64) * V)
        assert np.abs(rich[0, :, h] - ref).max() <= 1e-6 * np.abs(ref).max()


# ---------------------------------------------------------------- P6 exact write
def test_exact_write_invariant():
    """beta = 1 and |k_t| = 1: the decayed state is corrected so that S_t^T k_t = v_t exactly,
    for any decay. With q = k the output is therefore v. This holds only when the decay
    is applied before the erase and the erase has the minus sign."""
    q, k, v, g, beta, S0 = rand_case(6, T=20, H=3, dk=6, dv=4)
    kk = np.asarray(k, np.float64)
    k = (kk / np.linalg.norm(kk, axis=-1, keepdims=True)).astype(np.float32)
    k = k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True).astype(np.float32)
    beta[:] = 1
    o, _ = oracle.kda_reference(k, k, v, g, beta, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-5)


# ---------------------------------------------------------------- P7 orthonormal keys
def test_orthonormal_keys_reduce_to_linear_attention():
    """Orthonormal keys (T <= dk), beta = 1, g = 0, S0 = 0: nothing written earlier is
    erased, so KDA equals causal linear attention tril(Q K^T) V."""
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 8, 5
    Kq, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Kq[:T].astype(np.float32)[None, :, None, :]
    q = rng.standard_normal((1, T, 1, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    g = np.zeros((1, T, 1, dk), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    o, _ = oracle.kda_reference(q, k, v, g, beta)
    Q, K, V = (np.asarray(a[0, :, 0], np.float64) for a in (q, k, v))
    np.testing.assert_allclose(o[0, :, 0], np.tril(Q @ K.T) @ V, atol=1e-6)


# ---------------------------------------------------------------- P8 segments compose
def test_segment_composition_and_transition_form():
    """Running 0..T equals running T1..T from the state left at T1. And the P-way split of
    the infrastructure section: a segment's end state is M S0 + Z, with Z the zero-start
    state and M the transition (the segment run from S0 = I with v = 0, dv = dk);
    summing zero-start states instead is wrong."""
    q, k, v, g, beta, S0 = rand_case(8, T=24, H=2, dk=5, dv=3)
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    T1 = 10
    o1, s1 = oracle.kda_reference(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    o2, s2 = oracle.kda_reference(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-13)
    # transition form for the second segment
    sl = slice(T1, None)
    _, Z = oracle.kda_reference(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], None)
    dk = q.shape[-1]
    eye = np.broadcast_to(np.eye(dk), (1, q.shape[2], dk, dk)).copy()
    zeros_v = np.zeros(q[:, sl].shape, np.float32)
    _, M = oracle.kda_reference(q[:, sl], k[:, sl], zeros_v, g[:, sl], beta[:, sl], eye)
    np.testing.assert_allclose(np.einsum("nhab,nhbj->nhaj", M, s1) + Z, s, rtol=1e-11, atol=1e-12)
    # naive sum of zero-start states differs
    _, Z1 = oracle.kda_reference(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], None)
    _, Zall = oracle.kda_reference(q, k, v, g, beta, None)
    assert np.abs((Z1 + Z) - Zall).max() > 1e-2 * np.abs(Zall).max()


# ---------------------------------------------------------------- P9 varlen and batch
def test_varlen_and_batch_equal_independent_runs():
    q, k, v, g, beta, _ = rand_case(9, T=30, H=2, dk=4, dv=3)
    lens = [7, 1, 0, 13, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(9)
    S0 = rng.standard_normal((len(lens), 2, 4, 3))
    o, s = oracle.kda_reference(q, k, v, g, beta, S0, cu_seqlens=cu)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        oi, si = oracle.kda_reference(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                      S0[i:i + 1])
        np.testing.assert_array_equal(o[:, a:b], oi)
        np.testing.assert_array_equal(s[i], si[0])
    # dense batch of B rows = B independent sequences
    qb, kb, vb, gb, bb, Sb = rand_case(10, T=8, B=3)
    ob, sb = oracle.kda_reference(qb, kb, vb, gb, bb, Sb)
    for i in range(3):
        oi, si = oracle.kda_reference(qb[i:i + 1], kb[i:i + 1], vb[i:i + 1], gb[i:i + 1],
                                      bb[i:i + 1], Sb[i:i + 1])
        np.testing.assert_array_equal(ob[i], oi[0])
        np.testing.assert_array_equal(sb[i], si[0])


def test_chain_subset_matches_full_run():
    q, k, v, g, beta, S0 = rand_case(11, T=16, H=3)
    o, s = oracle.kda_reference(q, k, v, g, beta, S0)
    oc, sc = oracle.kda_reference(q, k, v, g, beta, S0, chains=[(0, 2), (0, 0)])
    for h in (0, 2):
        np.testing.assert_array_equal(oc[:, :, h], o[:, :, h])
        np.testing.assert_array_equal(sc[:, h], s[:, h])
    assert np.isnan(oc[:, :, 1]).all()


def test_decode_reference_is_one_token_recurrence():
    rng = np.random.default_rng(12)
    N, H, dk, dv = 5, 2, 4, 3
    q, k, v, g, beta, _ = rand_case(12, T=N, H=H, dk=dk, dv=dv, s0=False)
    S = rng.standard_normal((N, H, dk, dv))
    o, s = oracle.kda_decode_reference(q[0], k[0], v[0], g[0], beta[0], S)
    for n in range(N):
        on, sn = oracle.kda_reference(q[:, n:n + 1], k[:, n:n + 1], v[:, n:n + 1],
                                      g[:, n:n + 1], beta[:, n:n + 1], S[n:n + 1])
        np.testing.assert_array_equal(o[n], on[0, 0])
        np.testing.assert_array_equal(s[n], sn[0])


# ---------------------------------------------------------------- P10 the pages' numbers
def test_decay_floor_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "decay_floor_constants.json")))
    floor = inputs.GATE_FLOOR
    assert round(100 * math.exp(floor), 2) == c["retained_per_step_floor_percent"]
    lo, hi = c["tile_cumulative_log_decay_open_interval"]
    assert c["tile_tokens"] * floor == lo and hi == 0.0
    assert float(f"{math.exp(-lo):.1e}") == c["reciprocal_bound_printed"]
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert float(f"{bf16_max:.1e}") == c["bf16_range_printed"]
    # e^80 survives rounding to bf16 and e^-80 is a normal fp32 number
    e80 = inputs.round_to_bf16(np.array([math.exp(80.0)], np.float32))[0]
    assert np.isfinite(e80) and e80 < bf16_max
    assert np.float32(math.exp(-80.0)) > np.finfo(np.float32).tiny


@pytest.mark.parametrize("wid,T,H", [(0, None, None), (1, None, None), (2, 4096, 4),
                                     (3, 2048, 4)])
def test_generated_gates_respect_tile_bound(wid, T, H):
    x = inputs.make_prefill(wid, T=T, H=H)
    g = x.g.astype(np.float64)
    assert g.max() <= 0 and g.min() >= inputs.GATE_FLOOR
    Tn = g.shape[1] - g.shape[1] % 16
    tiles = g[:, :Tn].reshape(g.shape[0], Tn // 16, 16, *g.shape[2:]).sum(axis=2)
    assert tiles.min() >= 16 * inputs.GATE_FLOOR and tiles.max() <= 0
    if wid == 2:   # the adversarial half of the channels sits exactly on the floor
        assert (g == -5.0).mean() >= 0.5
        assert tiles.min() == -80.0


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(13).standard_normal(10000).astype(np.float32) * 100
    x[:4] = [-4.999, 1.0 / 3, 65504.0, 1e-30]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(inputs.round_to_bf16(x), ref)


# ---------------------------------------------------------------- P11 conditioning
def test_f32_oracle_close_to_f64():
    x = inputs.make_prefill(1, T=512, H=4)
    o64, s64 = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
    o32, s32 = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, precision="f32")
    assert np.abs(o32 - o64).max() <= 1e-5 * rms(o64)
    assert np.abs(s32 - s64).max() <= 1e-5 * rms(s64)


def test_state_size_independent_of_length():
    for T in (16, 64, 256):
        x = inputs.make_prefill(1, T=T, H=2)
        _, s = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
        assert s.shape == (1, 2, 128, 128)


def test_unbounded_inputs_break_the_tile_bound():
    """The ablation's inputs (g down to -20) leave the (-80, 0) tile range that the generated
    workloads respect, so they exercise exactly what the bound rules out."""
    from gated_delta_rule_59_amd import inputs
    x = inputs.make_unbounded(T=256, H=2)
    g = x.g.astype(np.float64)
    assert g.max() <= 0.0 and g.min() < -5.0
    tiles = g[0].reshape(16, 16, 2, 128).sum(axis=1)     # 16-token tile sums per channel
    assert tiles.min() < -80.0
