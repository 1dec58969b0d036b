"""Segmented walks of kda_chunk_fwd (the transition form of a sequence split) on the GPU.

With segments = P, each sequence's chunks are cut into P segments; the middle ones are first
summarised from zeros (Z) and from the identity with V = 0 (the transition Phi), the entry
states follow as entry_{p+1} = Phi_p entry_p + Z_p, and the segments are then walked from
their entries. Outputs, final states and checkpoints must match the oracle (which walks token
by token) and the sequential walk, for every segment count, ragged and empty segments."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, host, kda_inputs_dev
from tests.test_gpu_checkpoints import expected_checkpoints, ragged_case, seq_lengths

pytestmark = pytest.mark.gpu


def run(x, segments, **kw):
    import torch
    from gated_delta_rule_59_amd import binding
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    o, s = binding.chunk_fwd(q, k, v, g, beta, S0, cu, segments=segments, **kw)
    torch.cuda.synchronize()
    return host(o), host(s)


CASES = {
    "prefill-4k T=1024 H=2": lambda: inputs.make_prefill(1, T=1024, H=2),
    "prefill-64k-bound T=2048 H=2": lambda: inputs.make_prefill(2, T=2048, H=2),
    "5 chunks (empty trailing segments)": lambda: inputs.make_prefill(1, T=300, H=2),
    "ragged varlen": ragged_case,
    # weak decay: the segment transitions carry most of the state
    "long memory g>=-0.01 T=2048": lambda: inputs.make_long_memory(-0.01),
}


@pytest.mark.parametrize("segments", [3, 5, 8])
@pytest.mark.parametrize("name", list(CASES))
def test_segmented_walk_matches_oracle(name, segments):
    print(f"segments={segments}: {name}", flush=True)
    x = CASES[name]()
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens)
    o, s = run(x, segments)
    assert_parity(o, o_ref, TAU["bf16"], f"{name} o, {segments} segments")
    assert_parity(s, s_ref, TAU["bf16"], f"{name} S_T, {segments} segments")
    o1, s1 = run(x, 0)
    assert_parity(o, o1, TAU["bf16"], "segmented vs sequential o")


def test_segmented_checkpoints_in_place_no_s0():
    """Checkpoints across segment boundaries, the final state written over S0, and a zero
    initial state."""
    import torch
    from gated_delta_rule_59_amd import binding
    x = ragged_case()
    every = 64
    slots = binding.checkpoint_slots(seq_lengths(x), every)
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)
    ck = torch.full((slots, x.wl.H, 128, 128), float("nan"), device="cuda")
    S = S0.clone()
    binding.chunk_fwd(q, k, v, g, beta, S, cu, S_T=S, segments=4, ckpt=ck, ckpt_every=every)
    torch.cuda.synchronize()
    _, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens)
    assert_parity(host(S), s_ref, TAU["bf16"], "in-place final state, 4 segments")
    assert_parity(host(ck), expected_checkpoints(x, every), TAU["bf16"], "checkpoints, 4 segments")
    x.S0 = None
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, None, cu_seqlens=x.cu_seqlens)
    o, s = run(x, 6)
    assert_parity(o, o_ref, TAU["bf16"], "no S0 o, 6 segments")
    assert_parity(s, s_ref, TAU["bf16"], "no S0 S_T, 6 segments")


def test_long_sequence_few_heads():
    """The shape segmenting is for: one 65,536-token sequence with 2 heads (16 strip
    workgroups leave most of the GPU idle), decay at the floor on half the channels."""
    x = inputs.make_prefill(2, H=2)
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0)
    o, s = run(x, 8)
    assert np.isfinite(o).all()
    assert_parity(o, o_ref, TAU["bf16"], "long-2-heads o, 8 segments")
    assert_parity(s, s_ref, TAU["bf16"], "long-2-heads S_T, 8 segments")
