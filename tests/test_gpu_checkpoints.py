"""Sparse state checkpoints of kda_chunk_fwd (prefix reuse) on the GPU against the oracle.

Checkpoint j of sequence n must equal the final state of the oracle run on the first
j * every tokens of that sequence from the same S0[n]: all such prefixes are packed into one
varlen oracle call. Both prefill paths, dense and packed batches, ragged lengths, and a buffer
with fewer slots than checkpoints (the rest must stay untouched)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, host, kda_inputs_dev

pytestmark = pytest.mark.gpu


def seq_lengths(x):
    if x.cu_seqlens is None:
        return [x.wl.T] * x.wl.B
    return list(np.diff(x.cu_seqlens))


def expected_checkpoints(x, every):
    """Oracle states after every `every` tokens of each sequence, in slot order."""
    lens = seq_lengths(x)
    starts = [0] * len(lens) if x.cu_seqlens is None else list(x.cu_seqlens[:-1])
    rows = []   # (batch index, first token, prefix length, sequence)
    for n, L in enumerate(lens):
        for j in range(1, L // every + 1):
            b = n if x.cu_seqlens is None else 0
            rows.append((b, starts[n], j * every, n))
    if not rows:
        return np.zeros((0,) + x.S0.shape[1:], np.float64)
    pieces = [slice(t0, t0 + L) for (_, t0, L, _) in rows]
    cat = lambda a: np.concatenate([a[b, sl] for (b, _, _, _), sl in zip(rows, pieces)])[None]  # noqa: E731
    cu = np.concatenate([[0], np.cumsum([L for (_, _, L, _) in rows])]).astype(np.int32)
    S0 = np.stack([x.S0[n] for (_, _, _, n) in rows])
    _, s = oracle.kda_reference(cat(x.q), cat(x.k), cat(x.v), cat(x.g), cat(x.beta), S0,
                                cu_seqlens=cu)
    return s


def dense_case():
    B, T, H = 2, 300, 2
    q, k, v, g, beta = inputs.draw_activations((11, 1), B, T, H, 128, 128, "bf16")
    S0 = inputs.draw_state((11, 1), B, H, 128, 128)
    wl = inputs.Workload("ckpt-dense", 1, H, 128, 128, 64, "bf16", B=B, T=T)
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0)


def ragged_case():
    lens = [0, 1, 63, 64, 65, 137, 16, 300]
    T, H = sum(lens), 2
    q, k, v, g, beta = inputs.draw_activations((11, 2), 1, T, H, 128, 128, "bf16")
    S0 = inputs.draw_state((11, 2), len(lens), H, 128, 128)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    wl = inputs.Workload("ckpt-ragged", 3, H, 128, 128, 64, "bf16", B=1, T=T, lengths=lens,
                         n_seq=len(lens))
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0, cu)


@pytest.mark.parametrize("generic", [False, True], ids=["matrix-core", "fp32"])
@pytest.mark.parametrize("case,every", [("dense", 128), ("ragged", 64), ("ragged", 128)])
def test_checkpoints_match_prefix_states(case, every, generic):
    import torch
    from gated_delta_rule_59_amd import binding
    print(f"checkpoints: {case} every={every} generic={generic}", flush=True)
    x = dense_case() if case == "dense" else ragged_case()
    slots = binding.checkpoint_slots(seq_lengths(x), every)
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    ck = torch.full((slots + 1, x.wl.H, 128, 128), float("nan"), device="cuda")  # one spare
    o, s = binding.chunk_fwd(q, k, v, g, beta, S0, cu, generic=generic, ckpt=ck, ckpt_every=every)
    # the plain call takes the same walk steps: checkpoints between 128-token steps make the
    # matrix-core walk take one chunk per step, as walk64 does
    o_plain, s_plain = binding.chunk_fwd(q, k, v, g, beta, S0, cu, generic=generic,
                                         walk64=every % 128 != 0)
    torch.cuda.synchronize()
    want = expected_checkpoints(x, every)
    assert want.shape[0] == slots > 0
    got = host(ck)
    assert_parity(got[:slots], want, TAU["bf16"], f"checkpoints {case} every {every}")
    assert np.isnan(got[slots]).all()          # past the last checkpoint: untouched
    assert torch.equal(o, o_plain) and torch.equal(s, s_plain)   # outputs unaffected


def test_checkpoint_capacity_is_respected():
    """A buffer with fewer slots than checkpoints gets the first ones; nothing is written
    past its end."""
    import torch
    from gated_delta_rule_59_amd import binding
    x = ragged_case()
    every = 64
    slots = binding.checkpoint_slots(seq_lengths(x), every)
    cap = slots - 3
    big = torch.full((slots + 2, x.wl.H, 128, 128), float("nan"), device="cuda")
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    binding.chunk_fwd(q, k, v, g, beta, S0, cu, ckpt=big[:cap], ckpt_every=every)
    torch.cuda.synchronize()
    got = host(big)
    want = expected_checkpoints(x, every)
    assert_parity(got[:cap], want[:cap], TAU["bf16"], "checkpoints within capacity")
    assert np.isnan(got[cap:]).all()


def test_checkpoint_workload_prefill_4k():
    """prefill-4k at full size with a checkpoint every 512 tokens: all 16 heads, 8 states."""
    import torch
    from gated_delta_rule_59_amd import binding
    x = inputs.make_prefill(1)
    every = 512
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    ck = torch.empty((binding.checkpoint_slots(seq_lengths(x), every), x.wl.H, 128, 128),
                     device="cuda")
    binding.chunk_fwd(q, k, v, g, beta, S0, cu, ckpt=ck, ckpt_every=every)
    torch.cuda.synchronize()
    assert_parity(host(ck), expected_checkpoints(x, every), TAU["bf16"], "prefill-4k checkpoints")
