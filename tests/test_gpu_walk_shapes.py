"""Workgroup shapes and block formats of the matrix-core walk against the oracle. From the
number of (sequence, head) pairs the library picks 1, 2 or 4 strips of 16 state columns per
workgroup (four once there are at least four strips per CU, two from one per CU), and from one
strip per CU on the factored block (the walk forms U' = Utilde - W S per chunk). Each shape is
run here with its outputs in fp32 and bf16, run to run bitwise, final states, the pairwise
diagonal tiles, checkpoints, the final state written over S0, and a segmented walk."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_59_amd import inputs
from tests.gpu_util import TAU, assert_parity, host, kda_inputs_dev, rms
from tests.test_gpu_checkpoints import expected_checkpoints, seq_lengths

pytestmark = pytest.mark.gpu


def packed_case(n_seq, H, seed):
    lens = [int(x) for x in np.random.default_rng([0, 12, seed]).integers(0, 200, n_seq)]
    T = sum(lens)
    q, k, v, g, beta = inputs.draw_activations((12, seed), 1, T, H, 128, 128, "bf16")
    S0 = inputs.draw_state((12, seed), n_seq, H, 128, 128)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    wl = inputs.Workload(f"walk-shape-{n_seq}x{H}", 3, H, 128, 128, 64, "bf16", B=1, T=T,
                         lengths=lens, n_seq=n_seq)
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0, cu)


def dense_case(B, T, H, seed):
    q, k, v, g, beta = inputs.draw_activations((12, seed), B, T, H, 128, 128, "bf16")
    S0 = inputs.draw_state((12, seed), B, H, 128, 128)
    wl = inputs.Workload(f"walk-shape-dense-{B}x{T}x{H}", 1, H, 128, 128, 64, "bf16", B=B, T=T)
    return inputs.KDAInputs(wl, q, k, v, g, beta, S0)


def strips_per_workgroup(pairs, n_cu):
    """The launch-shape rule, restated: strips of one walk workgroup."""
    strips = pairs * 8
    return 4 if strips >= 4 * n_cu else 2 if strips >= n_cu else 1


# On a 256-CU GPU: 8 pairs (one strip, Psi/Z blocks); 40 and 42 pairs (two strips) and 160 pairs
# (four strips) with factored blocks, 42 leaving the last group of eight pairs part empty; a
# dense batch of 20 sequences of 150 tokens (40 pairs).
SHAPES = {"few pairs": lambda: packed_case(4, 2, 10), "two strips": lambda: packed_case(20, 2, 11),
          "42 pairs": lambda: packed_case(21, 2, 12), "four strips": lambda: packed_case(40, 4, 13),
          "dense 20 x 150": lambda: dense_case(20, 150, 2, 14)}


@pytest.mark.parametrize("name", list(SHAPES))
def test_walk_shapes(name):
    import torch
    from gated_delta_rule_59_amd import binding
    x = SHAPES[name]()
    H = x.wl.H
    n_seq = len(seq_lengths(x))
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    strips = strips_per_workgroup(n_seq * H, n_cu)
    print(f"{name}: {n_seq * H} pairs, {strips} strip(s) per workgroup on {n_cu} CUs, "
          f"{'factored' if strips >= 2 else 'Psi/Z'} blocks", flush=True)
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens)
    q, k, v, g, beta, S0, cu = kda_inputs_dev(x)

    # outputs and final state, one chunk per walk step so that checkpoints every 64 tokens
    # take the same walk
    o, s = binding.chunk_fwd(q, k, v, g, beta, S0, cu, walk64=True)
    o_again, s_again = binding.chunk_fwd(q, k, v, g, beta, S0, cu, walk64=True)
    torch.cuda.synchronize()
    assert_parity(host(o), o_ref, TAU["bf16"], f"{name} o")
    assert_parity(host(s), s_ref, TAU["bf16"], f"{name} S_T")
    assert torch.equal(o, o_again) and torch.equal(s, s_again)  # deterministic

    # bf16 outputs: at most half an ulp (2^-8 relative) more than the fp32-output error
    o16, _ = binding.chunk_fwd(q, k, v, g, beta, S0, cu, walk64=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got16 = host(o16)
    assert (np.abs(got16 - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + TAU["bf16"] * rms(o_ref)).all()

    # the diagonal tiles evaluated pairwise (the ablation's prep) feed the same walk
    o_pw, s_pw = binding.chunk_fwd(q, k, v, g, beta, S0, cu, walk64=True, pairwise_diag=True)
    torch.cuda.synchronize()
    assert_parity(host(o_pw), o_ref, TAU["bf16"], f"{name} o, pairwise diagonal tiles")
    assert_parity(host(s_pw), s_ref, TAU["bf16"], f"{name} S_T, pairwise diagonal tiles")

    # checkpoints every 64 tokens; the outputs are unaffected by them
    every = 64
    slots = binding.checkpoint_slots(seq_lengths(x), every)
    ck = torch.full((slots + 1, H, 128, 128), float("nan"), device="cuda")
    o2, s2 = binding.chunk_fwd(q, k, v, g, beta, S0, cu, ckpt=ck, ckpt_every=every)
    torch.cuda.synchronize()
    got = host(ck)
    assert_parity(got[:slots], expected_checkpoints(x, every), TAU["bf16"], f"{name} checkpoints")
    assert np.isnan(got[slots]).all()
    assert torch.equal(o2, o) and torch.equal(s2, s)

    # the final state written over S0 (one workgroup per walk)
    S = S0.clone()
    o3, _ = binding.chunk_fwd(q, k, v, g, beta, S, cu, S_T=S)
    torch.cuda.synchronize()
    assert_parity(host(S), s_ref, TAU["bf16"], f"{name} in place S_T")
    assert_parity(host(o3), o_ref, TAU["bf16"], f"{name} in place o")

    # a segmented walk of the same batch
    o4, s4 = binding.chunk_fwd(q, k, v, g, beta, S0, cu, segments=3)
    torch.cuda.synchronize()
    assert_parity(host(o4), o_ref, TAU["bf16"], f"{name} o, 3 segments")
    assert_parity(host(s4), s_ref, TAU["bf16"], f"{name} S_T, 3 segments")
