"""Helpers for the GPU tests: move generated inputs to the device and compare with the
oracle under the max-abs <= tau * RMS(reference) criterion."""
import numpy as np

TAU = {"bf16": 2e-2, "f32": 1e-4}


def rms(x):
    return float(np.sqrt(np.mean(np.square(np.asarray(x, np.float64)))))


def max_rel_err(got, ref, block=1 << 24):
    """max |got - ref| / RMS(ref) over the whole tensor, in blocks of `block` elements (the
    full-size workloads hold hundreds of millions of values)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1)
    r = ref.reshape(-1)
    worst, sq = 0.0, 0.0
    for a in range(0, g.size, block):
        gb = g[a:a + block].astype(np.float64)
        rb = r[a:a + block].astype(np.float64)
        assert np.isfinite(gb).all(), "non-finite values in GPU result"
        worst = max(worst, float(np.abs(gb - rb).max()))
        sq += float(np.dot(rb, rb))
    return worst / float(np.sqrt(sq / max(g.size, 1)))


def assert_parity(got, ref, tau, what):
    e = max_rel_err(got, ref)
    print(f"  parity {what}: max|err|/rms = {e:.3e} (tau {tau:g})", flush=True)
    assert e <= tau, f"{what}: max|err|/rms = {e:.3e} > {tau:g}"
    return e


def dev(x, dtype_name):
    """float32 numpy array holding values of dtype_name -> torch tensor on cuda (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype_name == "bf16" else t


def host(t):
    return t.float().cpu().numpy()


def kda_inputs_dev(x):
    """Device tensors of a KDAInputs (q, k, v, g, beta, S0, cu_seqlens)."""
    import torch
    d = x.wl.dtype
    out = [dev(a, d) for a in (x.q, x.k, x.v, x.g, x.beta)]
    out.append(None if x.S0 is None else torch.from_numpy(x.S0).to("cuda"))
    out.append(None if x.cu_seqlens is None else
               torch.from_numpy(x.cu_seqlens.astype(np.int32)).to("cuda"))
    return out
