"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill-4k]

A step is one kda_chunk_fwd (prefill: cumulative decay, tile products, the (I + A) inverse,
state propagation and outputs) over one batch of the workload, inputs already resident in
HBM. The headline workload (prefill-4k, B=1 H=16 T=4096) fits in the 256 MB last-level
cache, so it is timed cold: before each of the K timed launches, outside its HIP event pair, a
512 MiB buffer is read, which evicts inputs and workspace from L2 and the MALL. The
headline value is the tokens of one batch over the median of those K event times; the same
launch timed warm (K back-to-back launches inside one event pair) is a labelled secondary
figure. The long-context and packed workloads (prefill-64k-bound, varlen-16) are timed too,
each over 10 launches with an event pair per launch (their working sets are gigabytes, so
caches play no part), and the outputs of every timed workload are compared with the fp64
oracle over the whole tensors.

The decode half of the metric (GB/s against HBM peak) is measured in the same run: 1000
consecutive steps of the decode workload (N=512 sequences, H=32, 1 GiB fp32 state updated in
place), one event pair around all of them.

Secondary legs (checkpointed prefill, the pairwise-diagonal ablation, the segmented walk and
speculative verify/commit) are each timed over a window of at least 50 ms.

Prints ONE JSON line. The CPU oracle (its fp32 instantiation) is timed on a bounded sample of
the prefill and decode workloads as the reported CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16/fp16 matrix peak
WORKLOADS = {"prefill-4k": 1, "prefill-64k-bound": 2, "varlen-16": 3}
METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode GB/s % HBM peak (1 GPU)"
WINDOW_MS = 50.0              # minimum timed window of the secondary legs


def flops_per_token_head(C=64, d=128):
    """Algorithmic flops of the chunked forward per (token, head): A and Aqk (C d each), the
    triangular solve applied to both right-hand sides (2 C d), Aqk U' (C d), and the three
    state products (6 d^2)."""
    return 5 * C * d + 6 * d * d


def bytes_per_token_head(d=128, in_bytes=2, out_bytes=2):
    """Minimal bytes: q, k, g, v (d each) and beta read once, o written once. The default is
    the bf16-sized output; out_bytes=4 gives the count for the fp32 o the library writes."""
    return 4 * d * in_bytes + in_bytes + d * out_bytes


def state_bytes(n_seq, H, dk=128, dv=128):
    """S0 read once and S_T written once, fp32."""
    return 2 * 4 * dk * dv * n_seq * H


def src_hash(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_sources(*names):
    return [os.path.join(ROOT, "gated_delta_rule_59_amd", "csrc", n) for n in names]


PREFILL_SRC = ("kda_fast.hip", "kda_device.h", "kda_plan.h")
DECODE_SRC = ("kda_decode.hip", "kda_device.h")


def read_profile_value(profile_name, key, kernel_hash):
    """A figure from a committed rocprofv3 summary under profiles/, if the summary was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_src_sha") != kernel_hash:
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def read_traffic(profile_name, kernel_hash):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE)."""
    return read_profile_value(profile_name, "hbm_bytes_per_launch", kernel_hash)


def time_launches(fn, steps, warmup, stream):
    """Run fn() warmup times, then `steps` times between two synchronisations, with one HIP
    event pair on `stream` around all of them. Returns (wall seconds for the timed steps,
    average ms per launch from the events)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, a.elapsed_time(b) / steps


def time_window(fn, stream, min_ms=WINDOW_MS, min_launches=20):
    """Average event ms per launch over a window of at least min_ms (and min_launches
    launches), sized from a short first estimate. Returns (ms per launch, launches)."""
    _, est = time_launches(fn, 5, 3, stream)
    n = max(min_launches, int(math.ceil(min_ms / max(est, 1e-3))))
    _, ms = time_launches(fn, n, 0, stream)
    return ms, n


def time_each(fn, steps, stream, flush_bytes=0):
    """Event ms of each of `steps` launches (one event pair per launch, synchronised after
    each). With flush_bytes, a buffer of that size is read before each launch, outside its
    event pair, so that the launch starts with cold caches: the read evicts the inputs and
    the workspace from L2 and the 256 MB MALL and leaves clean lines behind (an overwrite
    would leave dirty ones for the launch to write back). Returns the sorted list."""
    import torch
    junk = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda") if flush_bytes else None
    ms = []
    for i in range(steps):
        if junk is not None:
            junk.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    return sorted(ms)


def median(xs):
    return xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] + xs[len(xs) // 2])


def oracle_threads():
    return int(os.environ.get("OMP_NUM_THREADS", 0)) or (os.cpu_count() or 1)


def parity(x, o, S_T):
    """max|err| / RMS(ref) of the timed o and S_T against the fp64 oracle over every chain of
    the workload (the whole tensors)."""
    import numpy as np
    import oracle
    threads = oracle_threads()
    t0 = time.perf_counter()
    o_ref, s_ref = oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0,
                                        cu_seqlens=x.cu_seqlens, threads=threads)
    el = time.perf_counter() - t0
    o = o.float().cpu().numpy()
    s = S_T.float().cpu().numpy()

    def rel(got, ref, block=1 << 24):   # in blocks: the long workloads hold ~1e9 values
        g, r = got.reshape(-1), ref.reshape(-1)
        worst, sq = 0.0, 0.0
        for a in range(0, g.size, block):
            gb, rb = g[a:a + block].astype(np.float64), r[a:a + block]
            d = np.abs(gb - rb).max()
            worst = float("nan") if not np.isfinite(d) else max(worst, float(d))
            sq += float(np.dot(rb, rb))
        return worst / math.sqrt(sq / max(g.size, 1))
    eo, es = rel(o, o_ref), rel(s, s_ref)
    tau = 2e-2
    return {"o_max_err_over_rms": eo, "S_T_max_err_over_rms": es, "tau": tau,
            "pass": bool(eo <= tau and es <= tau), "compared": "whole o and S_T",
            "oracle": f"fp64, {x.wl.n_seq * x.wl.H} chains on {threads} threads, {el:.1f} s "
                      "(timed apart from the baseline)"}


def cpu_baseline_prefill(x, budget_s):
    """The fp32 oracle (as committed) on the host cores: whole passes over the workload until
    budget_s has elapsed (at least one)."""
    import oracle
    threads = oracle_threads()
    chains = x.wl.n_seq * x.wl.H
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens,
                             precision="f32", threads=threads, want_state=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tokens = x.wl.B * x.wl.T
    return {"value": tokens * reps / el, "unit": "tokens/s", "cores": min(threads, chains),
            "kind": "oracle", "precision": "fp32",
            "sample": f"{reps} full pass(es) of {x.wl.name} (fp32 oracle, {chains} independent "
                      f"(sequence, head) chains over {threads} OpenMP threads, so at most "
                      f"{min(threads, chains)} cores busy), {el:.1f} s"}


def cpu_baseline_decode(S_host, pool, budget_s):
    """The fp32 oracle's decode step on the full decode state (all 16,384 chains), steps
    repeated until budget_s has elapsed (at least one)."""
    import numpy as np
    import oracle
    from gated_delta_rule_59_amd import inputs
    threads = oracle_threads()
    N, H, dk, dv = S_host.shape
    S = np.ascontiguousarray(S_host, dtype=np.float32)
    steps, t0 = 0, time.perf_counter()
    while True:
        _, S = oracle.kda_decode_reference(*pool[steps % inputs.DECODE_POOL], S, precision="f32",
                                           threads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / steps
    nbytes = N * H * (2 * 4 * dk * dv + 2 * (2 * dk + dk + dv + 1) + 4 * dv)
    return {"value": N / per, "unit": "tokens/s", "ms_per_step": per * 1e3,
            "GB_per_s": nbytes / per / 1e9, "cores": min(threads, N * H), "kind": "oracle",
            "precision": "fp32",
            "sample": f"{steps} step(s) of decode-512 (fp32 oracle over all {N * H} chains on "
                      f"{threads} OpenMP threads), {el:.1f} s"}


class Prefill:
    """Device tensors of one prefill workload and its launch."""

    def __init__(self, wid, stream):
        import torch
        from gated_delta_rule_59_amd import binding, inputs
        self.x = x = inputs.make_prefill(wid)
        self.stream = stream
        dv = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)  # noqa: E731
        self.q, self.k, self.v, self.g, self.beta = (dv(a) for a in (x.q, x.k, x.v, x.g, x.beta))
        self.S0 = torch.from_numpy(x.S0).cuda()
        self.cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens).cuda()
        self.B, self.T, self.H, self.d = x.q.shape
        self.n_seq = x.wl.n_seq if self.cu is not None else self.B
        self.o = torch.empty((self.B, self.T, self.H, self.d), dtype=torch.float32, device="cuda")
        self.S_T = torch.empty((self.n_seq, self.H, self.d, self.d), dtype=torch.float32,
                               device="cuda")
        self.ws_bytes = binding.chunk_fwd_workspace_bytes(self.q, self.k, self.v, self.g,
                                                          self.beta, self.S0, self.cu)
        self.ws = binding.alloc_workspace(self.ws_bytes, self.q.device)

    def launch(self, **kw):
        from gated_delta_rule_59_amd import binding
        binding.chunk_fwd(self.q, self.k, self.v, self.g, self.beta, self.S0, self.cu, o=self.o,
                          S_T=self.S_T, workspace=self.ws, stream=self.stream, **kw)

    def figures(self, ms):
        """Throughput and roofline figures of one launch taking `ms`."""
        token_heads = self.B * self.T * self.H
        flops = flops_per_token_head() * token_heads
        st = state_bytes(self.n_seq, self.H)
        b_min = bytes_per_token_head() * token_heads + st
        b_f32o = bytes_per_token_head(out_bytes=4) * token_heads + st
        sec = ms * 1e-3
        attainable = min(MFMA_PEAK_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9 * flops / b_min)
        return {"event_ms": ms, "tokens_per_s": self.B * self.T / sec,
                "alg_tflops": flops / sec / 1e12,
                "alg_mfma_frac": flops / sec / 1e12 / MFMA_PEAK_TFLOPS,
                "alg_GB_per_s": b_min / sec / 1e9, "alg_hbm_frac": b_min / sec / 1e9 / HBM_PEAK_GBS,
                "attainable_frac": (flops / sec) / attainable,
                "fp32_o_GB_per_s": b_f32o / sec / 1e9,
                "fp32_o_hbm_frac": b_f32o / sec / 1e9 / HBM_PEAK_GBS}

    def free(self):
        for name in ("q", "k", "v", "g", "beta", "S0", "cu", "o", "S_T", "ws"):
            setattr(self, name, None)


def roofline(fig, bytes_per_launch, traffic):
    return {"kernel": "kda_chunk_fwd launch (prep_kernel + the walk: rec_kernel, or rec_fact_kernel "
                      "with the factored block from 32 (sequence, head) pairs on)", "bound": "hbm",
            "achieved": fig["alg_GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": fig["alg_hbm_frac"], "traffic": traffic,
            "bytes_per_launch": bytes_per_launch,
            "bytes_count": "minimal: bf16 q, k, v, g, beta read once and a bf16-sized o written "
                           "once (1,282 B per token-head), plus S0 read and S_T written once; "
                           "fp32_o_* fields count the 4-byte o the library writes (1,538 B)"}


def bench_extra(name, stream, do_parity, launches=10):
    """A long prefill workload: event ms of each of `launches` launches (median, min), figures,
    traffic, parity."""
    import torch
    w = Prefill(WORKLOADS[name], stream)
    w.launch()
    w.launch()
    torch.cuda.synchronize()
    ms = time_each(w.launch, launches, stream)
    fig = w.figures(median(ms))
    fig["event_ms_min"] = ms[0]
    fig["launches"] = launches
    token_heads = w.B * w.T * w.H
    st = state_bytes(w.n_seq, w.H)
    out = {"workload": f"{name}: B={w.B} T={w.T} H={w.H} dk=dv=128 n_seq={w.n_seq}",
           "figures": fig, "workspace_bytes": w.ws_bytes,
           "roofline": roofline(fig, bytes_per_token_head() * token_heads + st,
                                read_traffic(f"{name}_chunk_fwd_traffic.txt",
                                             src_hash(*kernel_sources(*PREFILL_SRC))))}
    if do_parity:
        out["parity"] = parity(w.x, w.o, w.S_T)
    w.free()
    del w
    torch.cuda.empty_cache()
    return out


def bench_segments(stream):
    """The segmented walk on the shape it serves: one 65,536-token sequence with 2 heads
    (prefill-64k-bound's distributions), sequential and in 4 and 8 segments."""
    import torch
    from gated_delta_rule_59_amd import binding, inputs
    x = inputs.make_prefill(2, H=2)
    dv = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)  # noqa: E731
    q, k, v, g, beta = (dv(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    S0 = torch.from_numpy(x.S0).cuda()
    o = torch.empty(q.shape[:3] + (128,), dtype=torch.float32, device="cuda")
    S_T = torch.empty_like(S0)
    out = {"workload": "B=1 H=2 T=65536 dk=dv=128, decay floor on half the channels; the walk "
                       "takes 128-token composed steps (the default for so few pairs) unless "
                       "marked walk64"}
    for label, P, kw in (("sequential", 0, {}), ("sequential_walk64", 0, {"walk64": True}),
                         ("segments_4", 4, {}), ("segments_8", 8, {})):
        ws = binding.alloc_workspace(binding.chunk_fwd_workspace_bytes(q, k, v, g, beta, S0,
                                                                       segments=P, **kw),
                                     q.device)
        ms, n = time_window(lambda: binding.chunk_fwd(q, k, v, g, beta, S0, o=o, S_T=S_T,
                                                      workspace=ws, stream=stream, segments=P,
                                                      **kw), stream)
        out[f"{label}_event_ms"] = ms
        out[f"{label}_launches"] = n
    out["tokens_per_s_best"] = 65536 / (min(v for kk, v in out.items() if kk.endswith("_ms")) * 1e-3)
    return out


def bench_decode(steps, warmup, stream, cpu_budget):
    import torch
    from gated_delta_rule_59_amd import binding, inputs
    N, H, d = 512, 32, 128
    S_host = inputs.make_decode_state(N, H, d, d)
    S = torch.from_numpy(S_host).cuda()
    pool_host = [inputs.make_decode_step(p) for p in range(inputs.DECODE_POOL)]
    pool = [[torch.from_numpy(a).cuda().to(torch.bfloat16) for a in st] for st in pool_host]
    o = torch.empty((N, H, d), dtype=torch.float32, device="cuda")
    it = [0]

    def step():
        binding.decode_step(*pool[it[0] % inputs.DECODE_POOL], S, o=o, stream=stream)
        it[0] += 1

    wall, per = time_launches(step, steps, warmup, stream)
    nbytes = N * H * (2 * 4 * d * d + 2 * (4 * d + 1) + 4 * d)  # state in+out, inputs, fp32 o

    # speculative decoding on the same state: 4 draft tokens per sequence evaluated from one
    # read of S (verify, S untouched), then all 4 committed (S read and written, no outputs)
    m = 4
    drafts = [torch.from_numpy(a).cuda().to(torch.bfloat16)
              for a in inputs.draw_activations((0, 4, 1000), N, m, H, d, d, "bf16")]
    o_m = torch.empty((N, m, H, d), dtype=torch.float32, device="cuda")
    acc = torch.full((N,), m, dtype=torch.int32, device="cuda")
    v_ms, v_n = time_window(lambda: binding.decode_multi(*drafts, S, o=o_m, stream=stream), stream)
    c_ms, c_n = time_window(lambda: binding.decode_multi(*drafts, S, accept=acc,
                                                         want_output=False, stream=stream), stream)
    in_b = N * m * H * 2 * (4 * d + 1)
    spec = {"m": m, "verify_ms": v_ms, "verify_launches": v_n,
            "verify_tokens_per_s": N * m / (v_ms * 1e-3),
            "verify_GB_per_s": (N * H * 4 * d * d + in_b + N * m * H * 4 * d) / (v_ms * 1e-3) / 1e9,
            "commit_ms": c_ms, "commit_launches": c_n,
            "commit_GB_per_s": (N * H * 8 * d * d + in_b) / (c_ms * 1e-3) / 1e9}
    traffic = read_traffic("decode-512_decode_step_kernel_traffic.txt",
                           src_hash(*kernel_sources(*DECODE_SRC)))
    gbs = nbytes / (per * 1e-3) / 1e9
    res = {"workload": "decode-512 (N=512, H=32, dk=dv=128, fp32 state 1 GiB, bf16 inputs, "
                       "fp32 o), one step per launch, consecutive steps on the same state",
           "steps": steps, "warmup": warmup, "ms_per_step": per,
           "wall_ms_per_step": wall * 1e3 / steps,
           "tokens_per_s": N / (per * 1e-3), "GB_per_s": gbs, "spec_decode": spec,
           "roofline": {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": traffic, "bytes_per_launch": nbytes}}
    del S, pool, o, drafts, o_m
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline_decode(S_host, pool_host, cpu_budget)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed launches of the headline workload (cold, one event pair each)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill-4k", choices=list(WORKLOADS))
    ap.add_argument("--extra-workloads", default="prefill-64k-bound,varlen-16",
                    help="comma-separated prefill workloads timed besides the headline ('' = none)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-segments", action="store_true",
                    help="skip the segmented-walk timing on the long two-head sequence")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the checkpoint and pairwise-diagonal legs")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (scales HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: runs on one GPU only (asked for {args.gpus}); KDA "
              "prefill and decode shard over independent (sequence, head) pairs with no "
              "communication, so N GPUs would each run this same single-GPU workload.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "launches": 5}), flush=True)
        return
    from gated_delta_rule_59_amd import binding
    binding.lib()
    stream = torch.cuda.current_stream()
    phash = src_hash(*kernel_sources(*PREFILL_SRC))

    # ---- headline: cold launches of the headline workload
    w = Prefill(WORKLOADS[args.workload], stream)
    for _ in range(args.warmup):
        w.launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold = time_each(w.launch, args.steps, stream, flush_bytes=512 << 20)
    cold_wall = time.perf_counter() - t0
    head = w.figures(median(cold))
    head.update({"event_ms_min": cold[0], "event_ms_mean": sum(cold) / len(cold),
                 "launches": args.steps,
                 "timing": "cold: 512 MiB read before each launch, outside its event pair"})
    par = None if args.no_parity else parity(w.x, w.o, w.S_T)
    # warm secondary: back-to-back launches inside one event pair
    wall, warm_ms = time_launches(w.launch, args.steps, 0, stream)
    warm = w.figures(warm_ms)
    warm.update({"launches": args.steps, "wall_ms_per_launch": wall * 1e3 / args.steps,
                 "timing": "warm: back-to-back launches, one event pair around all (inputs and "
                           "workspace stay in L2 and the 256 MB MALL: not an HBM figure)"})
    token_heads = w.B * w.T * w.H
    bytes_min = bytes_per_token_head() * token_heads + state_bytes(w.n_seq, w.H)
    prefill = {
        "workload": f"{args.workload}: B={w.B} T={w.T} H={w.H} dk=dv=128 chunk 64 n_seq={w.n_seq}",
        "cold": head, "warm": warm, "parity": par, "workspace_bytes": w.ws_bytes,
        # executed matrix-core work (every MFMA issued, masked and repeated work included) as a
        # fraction of the matrix peak over the launch, from the committed SQ counter summary
        "rocprof_executed_mfma_busy_frac": read_profile_value(
            f"{args.workload}_sq_counters.txt", "mfma_busy_frac_launch", phash),
    }
    if not args.no_secondary:
        plain_ms, plain_n = time_window(w.launch, stream)
        ck_every = 512
        lens = [w.T] * w.B if w.cu is None else list(w.x.cu_seqlens[1:] - w.x.cu_seqlens[:-1])
        ck = torch.empty((binding.checkpoint_slots(lens, ck_every), w.H, w.d, w.d),
                         dtype=torch.float32, device="cuda")
        ck_ms, ck_n = time_window(lambda: w.launch(ckpt=ck, ckpt_every=ck_every), stream)
        pw_ms, pw_n = time_window(lambda: w.launch(pairwise_diag=True), stream)
        prefill["secondary_warm_window"] = {
            "plain_event_ms": plain_ms, "plain_launches": plain_n,
            "ckpt": {"every_tokens": ck_every, "slots": ck.shape[0], "event_ms": ck_ms,
                     "launches": ck_n, "overhead_vs_plain": ck_ms / plain_ms - 1.0},
            "pairwise_diag_ablation": {"event_ms": pw_ms, "launches": pw_n,
                                       "slowdown_vs_dense_diag": pw_ms / plain_ms}}
        del ck
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["event_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "T": w.T, "H": w.H, "dk": w.d,
                   "dv": w.d, "chunk": 64, "n_seq": w.n_seq, "inputs": "bf16 q/k/v/g/beta",
                   "state": "fp32", "output": "fp32", "global_batch": w.B, "seq_len": w.T,
                   "timing": "cold median of the timed launches",
                   "timed_region_wall_s": cold_wall},
        "roofline": roofline(head, bytes_min,
                             read_traffic(f"{args.workload}_chunk_fwd_traffic.txt", phash)),
        "prefill": prefill,
    }
    x_head = w.x
    w.free()
    del w
    torch.cuda.empty_cache()

    extra = [s for s in args.extra_workloads.split(",") if s and s != args.workload]
    if extra:
        res["prefill_workloads"] = {name: bench_extra(name, stream, not args.no_parity)
                                    for name in extra}
    if not args.no_segments:
        res["segments"] = bench_segments(stream)
    if not args.no_decode:
        res["decode"] = bench_decode(args.decode_steps, 3, stream,
                                     0 if args.no_cpu else args.cpu_budget)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_prefill(x_head, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
