"""kda_decode_multi (speculative decoding: evaluate m draft tokens, commit an accepted prefix)
on the GPU against the oracle.

Verification: the m outputs equal the oracle's outputs of an m-token sequence started from S,
and S is left bitwise unchanged. Commit: S becomes the oracle's state after the first
accept[n] tokens (0 and m included), and the outputs equal those of the verify call."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, dev, host, rms

pytestmark = pytest.mark.gpu


def draft_case(N, H, m, d, dtype, key):
    q, k, v, g, beta = inputs.draw_activations(key, N, m, H, d, d, dtype)
    S = inputs.draw_state(key, N, H, d, d)
    return q, k, v, g, beta, S


def oracle_after(q, k, v, g, beta, S, accept):
    """States after the first accept[n] tokens of each sequence (packed varlen call)."""
    N, m = q.shape[:2]
    cat = lambda a: np.concatenate([a[n, :accept[n]] for n in range(N)])[None]  # noqa: E731
    cu = np.concatenate([[0], np.cumsum(accept)]).astype(np.int32)
    _, s = oracle.kda_reference(cat(q), cat(k), cat(v), cat(g), cat(beta), S, cu_seqlens=cu)
    return s


# d = 128 with 2..8 drafts takes the one-pass kernel (register sizes 4 and 8, padded when m is
# smaller); one draft, more than eight, and other head sizes take the token loop
@pytest.mark.parametrize("N,H,m,d,dtype", [(48, 4, 5, 128, "bf16"), (8, 2, 3, 64, "bf16"),
                                           (6, 2, 4, 32, "f32"), (32, 4, 2, 128, "bf16"),
                                           (20, 3, 4, 128, "bf16"), (16, 2, 8, 128, "f32"),
                                           (12, 2, 3, 128, "f32"), (8, 2, 9, 128, "bf16")])
def test_verify_then_commit(N, H, m, d, dtype):
    import torch
    from gated_delta_rule_59_amd import binding
    print(f"spec decode N={N} H={H} m={m} d={d} {dtype}", flush=True)
    q, k, v, g, beta, S = draft_case(N, H, m, d, dtype, (21, N, m, d))
    tq, tk, tv, tg, tb = (dev(a, dtype) for a in (q, k, v, g, beta))
    tS = torch.from_numpy(S).cuda()
    S_before = tS.clone()
    o_v = binding.decode_multi(tq, tk, tv, tg, tb, tS)          # verify
    torch.cuda.synchronize()
    assert torch.equal(tS, S_before)
    o_ref, _ = oracle.kda_reference(q, k, v, g, beta, S)       # dense batch: N sequences of m
    tau = TAU[dtype]
    assert_parity(host(o_v), o_ref, tau, "draft outputs")
    rng = np.random.default_rng([21, N, m])
    acc = rng.integers(0, m + 1, size=N).astype(np.int32)
    acc[0], acc[-1] = 0, m
    o_c = binding.decode_multi(tq, tk, tv, tg, tb, tS, accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_v)
    s_ref = oracle_after(q, k, v, g, beta, S, acc)
    assert_parity(host(tS), s_ref, tau, "committed states")
    assert torch.equal(tS[0], S_before[0])                      # accept 0 leaves S alone


def test_commit_without_outputs_and_single_token():
    """A commit that skips the outputs gives the same state; m = 1 with every token accepted
    is one ordinary decode step."""
    import torch
    from gated_delta_rule_59_amd import binding
    N, H, m, d = 16, 2, 4, 128
    q, k, v, g, beta, S = draft_case(N, H, m, d, "bf16", (22, 1))
    tq, tk, tv, tg, tb = (dev(a, "bf16") for a in (q, k, v, g, beta))
    acc = torch.full((N,), 3, dtype=torch.int32, device="cuda")
    S1 = torch.from_numpy(S).cuda()
    S2 = S1.clone()
    binding.decode_multi(tq, tk, tv, tg, tb, S1, accept=acc)
    assert binding.decode_multi(tq, tk, tv, tg, tb, S2, accept=acc, want_output=False) is None
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    S3 = torch.from_numpy(S).cuda()
    S4 = S3.clone()
    one = torch.ones((N,), dtype=torch.int32, device="cuda")
    o_m = binding.decode_multi(tq[:, :1].contiguous(), tk[:, :1].contiguous(),
                               tv[:, :1].contiguous(), tg[:, :1].contiguous(),
                               tb[:, :1].contiguous(), S3, accept=one)
    o_s = binding.decode_step(tq[:, 0].contiguous(), tk[:, 0].contiguous(), tv[:, 0].contiguous(),
                              tg[:, 0].contiguous(), tb[:, 0].contiguous(), S4)
    torch.cuda.synchronize()
    assert torch.equal(o_m[:, 0], o_s) and torch.equal(S3, S4)


def test_spec_decode_workload_size():
    """The decode-512 shape (N=512, H=32, 1 GiB state) with 4 draft tokens per sequence: all
    outputs, then a commit of a seeded accepted prefix, every chain checked."""
    import torch
    from gated_delta_rule_59_amd import binding
    N, H, m, d = 512, 32, 4, 128
    q, k, v, g, beta = inputs.draw_activations((23, 1), N, m, H, d, d, "bf16")
    S = inputs.make_decode_state(N, H, d, d)
    tq, tk, tv, tg, tb = (dev(a, "bf16") for a in (q, k, v, g, beta))
    tS = torch.from_numpy(S).cuda()
    o = binding.decode_multi(tq, tk, tv, tg, tb, tS)
    acc = np.random.default_rng([23, 2]).integers(0, m + 1, size=N).astype(np.int32)
    binding.decode_multi(tq, tk, tv, tg, tb, tS, accept=torch.from_numpy(acc).cuda(),
                         want_output=False)
    torch.cuda.synchronize()
    o_ref, _ = oracle.kda_reference(q, k, v, g, beta, S)
    assert_parity(host(o), o_ref, TAU["bf16"], "decode-512 draft outputs")
    assert_parity(host(tS), oracle_after(q, k, v, g, beta, S, acc), TAU["bf16"],
                  "decode-512 committed states")


@pytest.mark.parametrize("m", [2, 4, 7])
def test_bf16_outputs_and_accept_clamped(m):
    """bf16 outputs (within half a bf16 ulp of the oracle plus the bar) from verify and commit,
    bitwise equal to each other; accept values below 0 or above m act as 0 and m."""
    import torch
    from gated_delta_rule_59_amd import binding
    N, H, d = 24, 2, 128
    print(f"spec decode bf16 out, clamped accept: m={m}", flush=True)
    q, k, v, g, beta, S = draft_case(N, H, m, d, "bf16", (24, m))
    tq, tk, tv, tg, tb = (dev(a, "bf16") for a in (q, k, v, g, beta))
    tS = torch.from_numpy(S).cuda()
    o_v = binding.decode_multi(tq, tk, tv, tg, tb, tS, out_dtype=torch.bfloat16)
    acc = np.random.default_rng([24, m]).integers(-2, m + 3, size=N).astype(np.int32)
    acc[:4] = [-5, 0, m, m + 7]
    o_c = binding.decode_multi(tq, tk, tv, tg, tb, tS, accept=torch.from_numpy(acc).cuda(),
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_v)
    o_ref, _ = oracle.kda_reference(q, k, v, g, beta, S)
    bound = 2.0 ** -8 * np.abs(o_ref) + TAU["bf16"] * rms(o_ref)
    assert (np.abs(host(o_v) - o_ref) <= bound).all()
    kept = np.clip(acc, 0, m)
    assert_parity(host(tS), oracle_after(q, k, v, g, beta, S, kept), TAU["bf16"],
                  "committed states, clamped accept")
