"""libkda: Kimi Delta Attention (KDA) chunked prefill and decode on AMD MI355X (gfx950).

The computation lives in the HIP kernels of csrc/, behind the C ABI declared in
include/kda.h; `binding` marshals torch tensors into it. `inputs` makes the seeded
synthetic workloads. Importing the package does not load the library; the first call does,
and fails loudly if it has not been built (python -m gated_delta_rule_59_amd.build).
"""
__all__ = ["chunk_fwd", "decode_step", "check_gates", "chunk_fwd_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
