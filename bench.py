"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill-4k]

A step is one kda_chunk_fwd (prefill: cumulative decay, tile products, the (I + A)
inverse, state propagation and outputs) over one batch of the workload, inputs already
resident on the GPU. K steps are timed between two device synchronisations, and bracketed
as a whole by a pair of HIP events on the stream they run on (the average launch duration is
the event time over K; no event sits between launches). A further --cold-steps launches
are timed one by one after a cache flush each (secondary figure). The decode half of the metric
(GB/s against HBM peak) is measured in the same run on the decode workload (N=512
sequences, H=32, 1 GiB fp32 state updated in place), from its own timed loop.

Prints ONE JSON line. The CPU oracle is timed on a bounded sample of the same workload
as the reported CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16/fp16 matrix peak
WORKLOADS = {"prefill-4k": 1, "prefill-64k-bound": 2, "varlen-16": 3}


def flops_per_token_head(C=64, d=128):
    """Algorithmic flops of the chunked forward per (token, head): A and Aqk (C d each), the
    triangular solve applied to both right-hand sides (2 C d), Aqk U' (C d), and the three
    state products (6 d^2)."""
    return 5 * C * d + 6 * d * d


def bytes_per_token_head(d=128, in_bytes=2, out_bytes=4):
    """q, k, g, v (d each) and beta read once; o written once."""
    return 4 * d * in_bytes + in_bytes + d * out_bytes


def src_hash(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def time_cold(fn, steps, stream, flush_bytes=512 << 20):
    """Per-launch event times with the caches cold: before each launch, outside its event
    pair, a 512 MiB buffer is overwritten, which evicts the inputs and the workspace from
    L2 and the 256 MB MALL. Returns (median ms, min ms)."""
    import torch
    junk = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    ms = []
    for i in range(steps):
        junk.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2], ms[0]


def cpu_baseline(x, budget_s=10.0):
    """The oracle (fp64, as committed) on the host cores: whole passes over the workload
    until budget_s has elapsed (at least one)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or (os.cpu_count() or 1)
    chains = x.wl.n_seq * x.wl.H
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.kda_reference(x.q, x.k, x.v, x.g, x.beta, x.S0, cu_seqlens=x.cu_seqlens,
                             threads=threads, want_state=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tokens = x.wl.B * x.wl.T
    return {"value": tokens * reps / el, "unit": "tokens/s", "cores": min(threads, chains),
            "kind": "oracle",
            "sample": f"{reps} full pass(es) of {x.wl.name} (fp64 oracle, {chains} independent "
                      f"(sequence, head) chains over {threads} OpenMP threads), {el:.1f} s"}


def bench_segments(stream, warmup, steps=10):
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
    out = {"workload": "B=1 H=2 T=65536 dk=dv=128, decay floor on half the channels"}
    for P in (0, 4, 8):
        ws = binding.alloc_workspace(binding.chunk_fwd_workspace_bytes(q, k, v, g, beta, S0,
                                                                       segments=P), q.device)
        _, ms = time_launches(lambda: binding.chunk_fwd(q, k, v, g, beta, S0, o=o, S_T=S_T,
                                                        workspace=ws, stream=stream,
                                                        segments=P), steps, max(2, warmup // 4),
                              stream)
        out[f"segments_{P}_event_ms" if P else "sequential_event_ms"] = ms
    out["tokens_per_s_best"] = 65536 / (min(v for kk, v in out.items() if kk.endswith("_ms")) * 1e-3)
    return out


def bench_decode(steps, warmup, stream):
    import torch
    from gated_delta_rule_59_amd import binding, inputs
    N, H, d = 512, 32, 128
    S = torch.from_numpy(inputs.make_decode_state(N, H, d, d)).cuda()
    pool = [[torch.from_numpy(a).cuda().to(torch.bfloat16) for a in inputs.make_decode_step(p)]
            for p in range(inputs.DECODE_POOL)]
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
    n_sp = max(10, steps // 4)
    _, ms_v = time_launches(lambda: binding.decode_multi(*drafts, S, o=o_m, stream=stream),
                            n_sp, 3, stream)
    _, ms_c = time_launches(lambda: binding.decode_multi(*drafts, S, accept=acc,
                                                         want_output=False, stream=stream),
                            n_sp, 3, stream)
    v_ms, c_ms = ms_v, ms_c
    in_b = N * m * H * 2 * (4 * d + 1)
    spec = {"m": m, "verify_ms": v_ms, "verify_tokens_per_s": N * m / (v_ms * 1e-3),
            "verify_GB_per_s": (N * H * 4 * d * d + in_b + N * m * H * 4 * d) / (v_ms * 1e-3) / 1e9,
            "commit_ms": c_ms, "commit_GB_per_s": (N * H * 8 * d * d + in_b) / (c_ms * 1e-3) / 1e9}
    ksrc = os.path.join(ROOT, "gated_delta_rule_59_amd", "csrc", "kda_decode.hip")
    traffic = read_traffic("decode-512_decode_step_kernel_traffic.txt", src_hash(ksrc))
    gbs = nbytes / (per * 1e-3) / 1e9
    return {"workload": "decode-512 (N=512, H=32, dk=dv=128, fp32 state 1 GiB, bf16 inputs, "
                        "fp32 o)",
            "steps": steps, "warmup": warmup, "ms_per_step": per,
            "wall_ms_per_step": wall * 1e3 / steps,
            "tokens_per_s": N / (per * 1e-3), "GB_per_s": gbs, "spec_decode": spec,
            "roofline": {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill-4k", choices=list(WORKLOADS))
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra launches timed after a 512 MiB cache flush each (0 = skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-segments", action="store_true",
                    help="skip the segmented-walk timing on the long two-head sequence")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (scales HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); KDA "
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
    from gated_delta_rule_59_amd import binding, inputs
    binding.lib()
    wid = WORKLOADS[args.workload]
    x = inputs.make_prefill(wid)
    stream = torch.cuda.current_stream()
    dv = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)  # noqa: E731
    q, k, v, g, beta = (dv(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    S0 = torch.from_numpy(x.S0).cuda()
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens).cuda()
    B, T, H, d = x.q.shape
    n_seq = x.wl.n_seq if cu is not None else B
    o = torch.empty((B, T, H, d), dtype=torch.float32, device="cuda")
    S_T = torch.empty((n_seq, H, d, d), dtype=torch.float32, device="cuda")
    nbytes_ws = binding.chunk_fwd_workspace_bytes(q, k, v, g, beta, S0, cu)
    ws = binding.alloc_workspace(nbytes_ws, q.device)

    def step():
        binding.chunk_fwd(q, k, v, g, beta, S0, cu, o=o, S_T=S_T, workspace=ws, stream=stream)

    wall, per_ms = time_launches(step, args.steps, args.warmup, stream)
    cold = time_cold(step, args.cold_steps, stream) if args.cold_steps else None
    # the same launch also storing the state every 512 tokens (sparse checkpoints)
    ck_every = 512
    lens = [T] * B if cu is None else list(x.cu_seqlens[1:] - x.cu_seqlens[:-1])
    ck = torch.empty((binding.checkpoint_slots(lens, ck_every), H, d, d), dtype=torch.float32,
                     device="cuda")

    def step_ck():
        binding.chunk_fwd(q, k, v, g, beta, S0, cu, o=o, S_T=S_T, workspace=ws, stream=stream,
                          ckpt=ck, ckpt_every=ck_every)

    _, ck_ms = time_launches(step_ck, max(10, args.steps // 4), 3, stream)
    # ablation: the same launch with the diagonal tiles evaluated pairwise (what the decay
    # bound's dense diagonal tiles save)
    _, pw_ms = time_launches(lambda: binding.chunk_fwd(q, k, v, g, beta, S0, cu, o=o, S_T=S_T,
                                                       workspace=ws, stream=stream,
                                                       pairwise_diag=True),
                             max(10, args.steps // 4), 3, stream)
    token_heads = B * T * H
    flops = flops_per_token_head() * token_heads
    nbytes = bytes_per_token_head() * token_heads + 2 * 4 * d * d * n_seq * H
    gbs = nbytes / (per_ms * 1e-3) / 1e9
    tflops = flops / (per_ms * 1e-3) / 1e12
    ksrc = [os.path.join(ROOT, "gated_delta_rule_59_amd", "csrc", f)
            for f in ("kda_fast.hip", "kda_device.h")]
    traffic = read_traffic(f"{args.workload}_chunk_fwd_traffic.txt", src_hash(*ksrc))
    # executed matrix-core work (every MFMA issued, masked and repeated work included) as a
    # fraction of the matrix peak over the launch, from the committed SQ counter summary
    mfma_busy = read_profile_value(f"{args.workload}_sq_counters.txt", "mfma_busy_frac_launch",
                                   src_hash(*ksrc))
    tokens = B * T
    # the roofline ceiling for this path: min(matrix peak, HBM peak x flops per byte)
    attainable = min(MFMA_PEAK_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9 * flops / nbytes)
    res = {
        "metric": "KDA prefill tokens/s + % bf16 MFMA peak; decode GB/s % HBM peak (1 GPU)",
        "value": tokens / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": x.wl.name, "B": B, "T": T, "H": H, "dk": d, "dv": d,
                   "chunk": 64, "n_seq": n_seq, "inputs": "bf16 q/k/v/g/beta",
                   "state": "fp32", "output": "fp32", "global_batch": B, "seq_len": T},
        "prefill": {"event_ms_per_launch": per_ms, "tokens_per_s_event": tokens / (per_ms * 1e-3),
                    "alg_tflops": tflops, "alg_mfma_frac": tflops / MFMA_PEAK_TFLOPS,
                    "alg_GB_per_s": gbs, "alg_hbm_frac": gbs / HBM_PEAK_GBS,
                    "attainable_frac": (flops / (per_ms * 1e-3)) / attainable,
                    "rocprof_executed_mfma_busy_frac": mfma_busy,
                    "workspace_bytes": nbytes_ws,
                    "cold_event_ms_median": cold and cold[0], "cold_event_ms_min": cold and cold[1],
                    "cold_steps": args.cold_steps,
                    "ckpt": {"every_tokens": ck_every, "slots": ck.shape[0],
                             "event_ms_per_launch": ck_ms,
                             "overhead_vs_plain": ck_ms / per_ms - 1.0},
                    "pairwise_diag_ablation": {"event_ms_per_launch": pw_ms,
                                               "slowdown_vs_dense_diag": pw_ms / per_ms}},
        "roofline": {"kernel": "kda_chunk_fwd launch (prep_kernel + rec_kernel)", "bound": "hbm",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
    }
    if not args.no_segments:
        res["segments"] = bench_segments(stream, args.warmup)
    if not args.no_decode:
        res["decode"] = bench_decode(args.decode_steps, max(3, args.warmup // 4), stream)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
