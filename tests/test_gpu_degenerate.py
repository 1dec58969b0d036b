"""Degenerate gates on the GPU, through the C ABI, against the oracle and against the closed
forms the recurrence reduces to:
  - beta = 0: nothing is written, the state only decays, so S_T = Diag(e^{G_T}) S0 and
    o_t = (Diag(e^{G_t}) S0)^T q_t (G_t the cumulative log-decay up to and including t);
  - beta = 0 and g = 0: the state passes through unchanged (bitwise) and o_t = S0^T q_t;
  - g = 0: no decay, the plain delta rule;
  - beta = 1 with keys of exactly unit norm: the write is exact, S_t^T k_t = v_t for every t
    and any g (the decayed state's prediction of v_t is replaced by v_t itself);
  - g = -5 on every key channel: every 16-token tile's cumulative log-decay is exactly -80,
    the edge of the range the decay bound guarantees;
  - gates of mixed magnitude (-5, -1e-3, -1e-6 and 0 at random per element): the per-tile
    prefix sums add terms six orders of magnitude apart.
Both prefill paths (the matrix-core path and the fp32 path), the decode step and speculative
drafts are covered."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, host, kda_inputs_dev, rms

pytestmark = pytest.mark.gpu

T, H = 333, 2   # six chunks, the last one partial


def _unit_keys(x, seed=11):
    """Replace k by keys of exactly unit norm in bf16: +-1/8 on a random half of the 128
    channels (64 * (1/8)^2 = 1, every value exact in bf16)."""
    rng = np.random.default_rng([0, 7, seed])
    B, Tn, Hn, dk = x.k.shape
    k = np.zeros((B, Tn, Hn, dk), np.float32)
    for idx in np.ndindex(B, Tn, Hn):
        ch = rng.choice(dk, dk // 2, replace=False)
        k[idx + (ch,)] = rng.choice([-0.125, 0.125], dk // 2)
    x.k = k
    return x


def beta0():
    x = inputs.make_long_memory(-0.01, T=T, H=H)   # weak decay: S0 stays visible in o
    x.beta = np.zeros_like(x.beta)
    return x


def identity():
    x = inputs.make_prefill(1, T=T, H=H)
    x.beta = np.zeros_like(x.beta)
    x.g = np.zeros_like(x.g)
    return x


def g0():
    x = inputs.make_prefill(1, T=T, H=H)
    x.g = np.zeros_like(x.g)
    return x


def beta1():
    x = _unit_keys(inputs.make_prefill(1, T=T, H=H))
    x.beta = np.ones_like(x.beta)
    return x


def floor():
    x = inputs.make_prefill(1, T=T, H=H)
    x.g = np.full_like(x.g, inputs.GATE_FLOOR)
    return x


def mixed():
    x = inputs.make_prefill(1, T=T, H=H)
    rng = np.random.default_rng([0, 7, 12])
    levels = np.array([inputs.GATE_FLOOR, -1e-3, -1e-6, 0.0], np.float32)
    x.g = inputs.round_to_bf16(levels[rng.integers(0, 4, x.g.shape)])
    return x


CASES = {"beta=0": beta0, "beta=0 g=0": identity, "g=0": g0, "beta=1 unit k": beta1,
         "g=-5 everywhere": floor, "mixed magnitudes": mixed}


def run(x, generic):
    import torch
    from gated_delta_rule_59_amd import binding
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    o, s = binding.chunk_fwd(q, k, v, g, beta, S0, cu, generic=generic)
    torch.cuda.synchronize()
    return host(o), host(s)


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_matches_oracle(name, generic):
    print(f"degenerate {name} generic={generic}", flush=True)
    x = CASES[name]()
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
    o, s = run(x, generic)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert_parity(o, o_ref, TAU["bf16"], f"{name} o")
    assert_parity(s, s_ref, TAU["bf16"], f"{name} S_T")


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
def test_beta0_closed_form(generic):
    """beta = 0: the GPU's outputs and final state against the decay-only closed form,
    evaluated here in fp64 without the oracle."""
    x = beta0()
    o, s = run(x, generic)
    G = np.cumsum(x.g.astype(np.float64), axis=1)                     # [B, T, H, dk]
    S0 = x.S0.astype(np.float64)                                      # [B, H, dk, dv]
    o_cf = np.einsum("bthc,bhcv->bthv", x.q * np.exp(G), S0)
    s_cf = np.exp(G[:, -1])[..., None] * S0
    assert_parity(o, o_cf, TAU["bf16"], "beta=0 o vs closed form")
    assert_parity(s, s_cf, TAU["bf16"], "beta=0 S_T vs closed form")


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
def test_identity_passes_the_state_through(generic):
    """beta = 0 and g = 0: S_T is S0 bit for bit and o_t = S0^T q_t."""
    x = identity()
    o, s = run(x, generic)
    np.testing.assert_array_equal(s, x.S0)
    o_cf = np.einsum("bthc,bhcv->bthv", x.q.astype(np.float64), x.S0.astype(np.float64))
    assert_parity(o, o_cf, TAU["bf16"], "beta=0 g=0 o vs S0^T q")


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
def test_exact_write_with_unit_keys(generic):
    """beta = 1 and |k| = 1 exactly: after the last token, S_T^T k_T = v_T, for the recipe's
    decay (a property of the result alone, checked without the oracle)."""
    x = beta1()
    _, s = run(x, generic)
    pred = np.einsum("bhcv,bhc->bhv", s.astype(np.float64), x.k[:, -1].astype(np.float64))
    v_last = x.v[:, -1].astype(np.float64)
    assert_parity(pred, v_last, TAU["bf16"], "S_T^T k_T vs v_T")


def test_decode_degenerate_gates():
    """Decode step: beta = 0, g = 0 leaves S bitwise unchanged with o = S^T q; beta = 1 with
    unit keys makes the new state predict v exactly (S_new^T k = v)."""
    import torch
    from gated_delta_rule_59_amd import binding
    N, Hd = 8, 4
    q, k, v, g, beta = inputs.make_decode_step(3, N=N, H=Hd)
    S = inputs.make_decode_state(N, Hd)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(torch.bfloat16)  # noqa: E731

    Sd = torch.from_numpy(S).cuda()
    o = binding.decode_step(dev(q), dev(k), dev(v), dev(np.zeros_like(g)),
                            dev(np.zeros_like(beta)), Sd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Sd), S)
    assert_parity(host(o), np.einsum("nhc,nhcv->nhv", q.astype(np.float64), S.astype(np.float64)),
                  TAU["bf16"], "decode beta=0 g=0 o vs S^T q")

    rng = np.random.default_rng([0, 7, 99])
    ku = np.zeros_like(k)
    for idx in np.ndindex(N, Hd):
        ch = rng.choice(128, 64, replace=False)
        ku[idx + (ch,)] = rng.choice([-0.125, 0.125], 64)
    Sd = torch.from_numpy(S).cuda()
    o = binding.decode_step(dev(q), dev(ku), dev(v), dev(g), dev(np.ones_like(beta)), Sd)
    torch.cuda.synchronize()
    Sn = host(Sd).astype(np.float64)
    assert_parity(np.einsum("nhcv,nhc->nhv", Sn, ku.astype(np.float64)), v.astype(np.float64),
                  TAU["bf16"], "decode beta=1 S_new^T k vs v")
    o_ref, s_ref = oracle.kda_decode_reference(q, ku, v, g, np.ones_like(beta), S)
    assert_parity(host(o), o_ref, TAU["bf16"], "decode beta=1 o")
    assert_parity(host(Sd), s_ref, TAU["bf16"], "decode beta=1 S")


@pytest.mark.parametrize("m", [1, 4, 8])
def test_drafts_degenerate_gates(m):
    """Speculative drafts (one-pass kernel for m = 2..8, token loop for m = 1): beta = 0 and
    g = 0 make every draft's output S^T q_j and a commit of all drafts leave S bitwise
    unchanged; beta = 1 with unit keys makes the committed state predict the last draft's v
    exactly (S_new^T k = v)."""
    import torch
    from gated_delta_rule_59_amd import binding
    N, Hd, d = 8, 2, 128
    print(f"draft degenerate gates: m={m}", flush=True)
    q, k, v, g, beta = inputs.draw_activations((41, m), N, m, Hd, d, d, "bf16")
    S = inputs.draw_state((41, m), N, Hd, d, d)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    all_in = torch.full((N,), m, dtype=torch.int32, device="cuda")

    Sd = torch.from_numpy(S).cuda()
    o = binding.decode_multi(dv(q), dv(k), dv(v), dv(np.zeros_like(g)), dv(np.zeros_like(beta)),
                             Sd, accept=all_in)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Sd), S)
    o_ref = np.einsum("nmhc,nhcv->nmhv", q.astype(np.float64), S.astype(np.float64))
    assert_parity(host(o), o_ref, TAU["bf16"], "drafts beta=0 g=0 o vs S^T q")

    rng = np.random.default_rng([0, 7, 100 + m])
    ku = np.zeros_like(k)
    for idx in np.ndindex(N, m, Hd):
        ch = rng.choice(d, 64, replace=False)
        ku[idx + (ch,)] = rng.choice([-0.125, 0.125], 64)
    Sd = torch.from_numpy(S).cuda()
    binding.decode_multi(dv(q), dv(ku), dv(v), dv(g), dv(np.ones_like(beta)), Sd, accept=all_in,
                         want_output=False)
    torch.cuda.synchronize()
    Sn = host(Sd).astype(np.float64)
    pred = np.einsum("nhcv,nhc->nhv", Sn, ku[:, -1].astype(np.float64))
    assert_parity(pred, v[:, -1].astype(np.float64), TAU["bf16"], "drafts beta=1 S_new^T k_last vs v_last")
