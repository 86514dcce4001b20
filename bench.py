"""RACE Attention layer benchmark on one MI355X.

One step = forward + backward of the whole RACE MHA layer core (all heads)
over one batch of synthetic input already resident in HBM: race_attn_fwd
(keeping the per-chunk sketch states and per-token denominators) then
race_attn_bwd (reusing them with O).

Default workload: causal, B=1, H=4, N=12,000,000, d=64, P=4, L=16,
chunk=1024, bf16 inputs with float32 sketches; Q, K, V, dO iid N(0,1) from
the seeded Philox stream. Prints ONE JSON line. After the timed layer steps
(outside their timed region) it also times race_attn_decode, one token per
head against the running sketch, at the same head shape ("decode").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12           # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}   # dense matrix FLOP/s

COPY_BYTES = 1 << 30        # reference copy: reads and writes this many bytes
METRIC = "RACE MHA layer fwd+bwd tokens/s (causal, N=12M) + % of HBM/MFMA roofline"


def per_token_head_counts(w):
    """Algorithmic bytes and FLOPs per (batch, head, token), d = 64.

    Layer: forward reads Q, K, V and writes O; backward reads Q, K, V, dO and
    writes dQ, dK, dV. FLOPs: forward 4 d L P (two projections) + 2 U (one
    sketch-sized contraction to read out, one to write), backward 8 d L P + 4 U,
    with U = 2 L R (d + 1).
    Per kernel: the layer tensors it reads or writes (each once; the stored
    plane values, O, D, e and the chunk states are implementation overhead)
    and its own contractions:
      totals_kv  : K, V in;                    2dLP (projection) + U
      pass_fwd   : Q, V in, O out;             2dLP (projection) + 2U
      pass_bwd_q : Q, V, dO in, dQ out;        2dLP (back-projection) + 2U
      totals_qg  : dO in;                      U
      pass_bwd_v : dO in, dV out;              2U
      pass_bwd_k : K, V, dO in, dK out;        2dLP (back-projection) + 2U
    """
    es = 2 if w.dtype == "bf16" else 4
    row = w.d * es
    R = 1 << w.P
    U = 2 * w.L * R * (w.d + 1)
    dLP = w.d * w.L * w.P
    layer = {"bytes": 4 * row + 7 * row, "flops": (4 * dLP + 2 * U) + (8 * dLP + 4 * U)}
    kernels = {
        "totals_kv": (2 * row, 2 * dLP + U),
        "pass_fwd": (3 * row, 2 * dLP + 2 * U),
        "pass_bwd_q": (4 * row, 2 * dLP + 2 * U),
        "totals_qg": (1 * row, U),
        "pass_bwd_v": (2 * row, 2 * U),
        "pass_bwd_k": (4 * row, 2 * dLP + 2 * U),
    }
    return layer, kernels


TRAFFIC_DIR = os.path.join(ROOT, "profiles")


# Sources that decide what the kernels and their launches do (the C-ABI
# front end, race_abi.hip, only validates arguments and is left out).
KERNEL_SOURCES = ("race_device.hpp", "race_kernels.hpp", "race_decode.hpp", "race_dispatch.hpp",
                  "race_host.hpp", "race_bf16.hip", "race_f32.hip")


def source_digest() -> str:
    """sha256 over the kernel sources: identifies the build that HBM byte
    counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_lsh_sketch_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name not in KERNEL_SOURCES:
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` (FETCH_SIZE + WRITE_SIZE, each scaled by
    the same counter on a 1 GiB reference copy) from the committed summary
    profiles/hbm_traffic_<workload>.md, or None when there is none for this
    workload or it was taken on other kernel sources."""
    path = os.path.join(TRAFFIC_DIR, f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest, rows = None, {}
    for line in open(path):
        if line.startswith("sources sha256:"):
            digest = line.split(":", 1)[1].strip()
        elif line.startswith("| pass_") or line.startswith("| totals_") or line.startswith("| scan_"):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            try:
                rows[cells[0]] = int(cells[-1])
            except ValueError:
                pass
    if digest != source_digest():
        return None
    return rows.get(stage)


def copy_bandwidth(dev, nbytes: int = COPY_BYTES, reps: int = 5) -> float:
    """GB/s (bytes read + bytes written) of a plain device-to-device copy of
    nbytes on this machine: the attainable HBM rate, reported beside the nominal
    peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (s.elapsed_time(e) / 1e3) / 1e9
    del src, dst
    return gbps


def matmul_rate(dev, dtype, n: int = 8192, reps: int = 10) -> float:
    """TFLOP/s of a dense n x n x n matrix product in `dtype` (the BLAS
    library's matrix-core kernel) on this machine: the attainable matrix rate,
    reported beside the nominal peak."""
    import torch
    a = torch.randn((n, n), device=dev).to(dtype)
    b = torch.randn((n, n), device=dev).to(dtype)
    c = a @ b
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        c = a @ b
    e.record()
    torch.cuda.synchronize()
    tflops = 2 * n ** 3 * reps / (s.elapsed_time(e) / 1e3) / 1e12
    del a, b, c
    return tflops


def cpu_baseline(w, n_sample: int):
    """The float64 oracle on the first n_sample tokens of every head of the
    same workload (same seeded inputs), causal forward + backward."""
    import numpy as np
    import synth
    from oracle import stream as oracle

    shape = (w.B, w.H, n_sample, w.d)
    host = {}
    for name, tid in (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO)):
        arr = np.empty(shape, np.uint16 if w.dtype == "bf16" else np.float32)
        for b in range(w.B):
            for h in range(w.H):
                start = ((b * w.H + h) * w.N) * w.d
                arr[b, h] = synth.normal(w.seed, tid, (n_sample, w.d), w.dtype, start=start)
        host[name] = arr
    W = synth.normal(w.seed, synth.TID_W, (w.L, w.P, w.d), w.dtype)
    W64 = synth.bf16_bits_to_f64(W) if w.dtype == "bf16" else W.astype(np.float64)
    affinity = len(os.sched_getaffinity(0))
    omp_env = os.environ.get("OMP_NUM_THREADS")
    # the oracle runs one thread per (batch, head) sequence, at most the
    # OpenMP thread count the environment allows
    limit = affinity if omp_env is None else max(1, min(affinity, int(omp_env)))
    threads = min(w.B * w.H, limit)
    t0 = time.perf_counter()
    oracle.forward(host["Q"], host["K"], host["V"], W64, w.beta, w.causal)
    oracle.backward(host["Q"], host["K"], host["V"], W64, host["dO"], w.beta, w.causal)
    dt = time.perf_counter() - t0
    return {"value": w.B * n_sample / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_sample} tokens of each of the {w.B * w.H} (batch, head) sequences, "
                      f"causal fwd+bwd in float64, {dt:.1f} s",
            "affinity_cpus": affinity, "omp_num_threads": omp_env, "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# (heads, tokens per head and call): the long-context workload's 4 heads; 512
# sequences x 32 heads (1.1 GB of state, beyond the 256 MB last-level cache,
# so the rate is HBM's); 256 x 32 heads extending each sequence by 8 tokens
# per call (a draft to verify, a prompt piece)
DECODE_CASES = ((4, 1), (16384, 1), (8192, 8))


def decode_measure(w, dev, steps: int = 200):
    """Causal decode against the running sketch (race_attn_decode) at the
    workload's head shape: microseconds per call (T tokens for every head),
    launched one by one from Python and replayed from a HIP graph, and the
    state read-modify-write rate (of the launched calls) against the HBM
    peak. Algorithmic bytes per head and call: the sketch read and written
    once (2 * L * 2^P * (4 d + 8): float32 value sums, float64 masses) plus
    q, k, v in and o out per token."""
    import torch
    import linear_lsh_sketch_amd as race
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    W = torch.randn((w.L, w.P, w.d), generator=gen, device=dev).to(tdt)
    state_rw = 2 * w.L * (1 << w.P) * (w.d * 4 + 8)   # float32 value sums, float64 masses
    res = {"workload": f"decode_P{w.P}_L{w.L}_d{w.d}_{w.dtype}", "heads": [], "tokens_per_call": [],
           "us_per_call": [], "us_per_call_graph": [], "alg_bytes_per_head": [], "GBps": [], "frac_hbm": [],
           "tokens_per_s": [], "tokens_per_s_graph": []}
    for heads, T in DECODE_CASES:
        q, k, v = (torch.randn((heads, 1, T, w.d), generator=gen, device=dev).to(tdt) for _ in range(3))
        state = race.alloc_state(heads, 1, w.P, w.L, dev)
        o = torch.empty_like(q)
        for _ in range(5):
            race.decode(q, k, v, W, state, w.P, w.L, w.beta, out=o)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(steps):
            race.decode(q, k, v, W, state, w.P, w.L, w.beta, out=o)
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / steps
        # the same calls captured once in a HIP graph and replayed: no host
        # launch cost between them (how a serving loop would issue them)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                race.decode(q, k, v, W, state, w.P, w.L, w.beta, out=o)
        graph.replay()
        torch.cuda.synchronize()
        s.record()
        graph.replay()
        e.record()
        torch.cuda.synchronize()
        us_graph = s.elapsed_time(e) * 1e3 / steps
        del graph
        alg = state_rw + 4 * T * w.d * es
        gbps = heads * alg / (us * 1e-6) / 1e9
        res["heads"].append(heads)
        res["tokens_per_call"].append(T)
        res["us_per_call"].append(us)
        res["us_per_call_graph"].append(us_graph)
        res["alg_bytes_per_head"].append(alg)
        res["GBps"].append(gbps)
        res["frac_hbm"].append(gbps * 1e9 / HBM_PEAK)
        res["tokens_per_s"].append(heads * T / (us * 1e-6))
        res["tokens_per_s_graph"].append(heads * T / (us_graph * 1e-6))
        del q, k, v, state, o
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="causal_long_n12M")
    ap.add_argument("--chunk", type=int, default=0,
                    help="tokens per workgroup (default: the workload's); only for the non-causal "
                         "workload, whose chunk the configuration leaves free")
    ap.add_argument("--cpu-sample", type=int, default=262144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step measurement that follows the timed layer steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy before the steps (the reference "
                         "dispatch for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the sequence-sharded "
              "multi-GPU path is a design, not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_lsh_sketch_amd as race
    import synth
    from synth.workloads import BY_NAME

    w = BY_NAME[args.workload]
    if args.chunk:
        if w.causal:
            print("--chunk applies to the non-causal workload only (the causal ones fix it)", file=sys.stderr)
            sys.exit(2)
        import dataclasses
        w = dataclasses.replace(w, chunk=args.chunk)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = (w.B, w.H, w.N, w.d)
    t = {}
    for name, tid in (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO)):
        t[name] = torch.empty(shape, dtype=tdt, device=dev)
        if w.qk_dist == "mixture" and name in ("Q", "K"):
            synth.mixture_device(w.seed, tid, synth.TID_QIDS if name == "Q" else synth.TID_KIDS, t[name])
        else:
            synth.normal_device(w.seed, tid, t[name])
    t["W"] = synth.normal_device(w.seed, synth.TID_W, torch.empty((w.L, w.P, w.d), dtype=tdt, device=dev))
    O = torch.empty(shape, dtype=tdt, device=dev)
    grads = tuple(torch.empty(shape, dtype=tdt, device=dev) for _ in range(3))
    ws_f = race.alloc_workspace(w.B, w.H, w.N, w.P, w.L, w.causal, w.chunk, race.WS_FWD_SAVED, dev)
    ws_b = race.alloc_workspace(w.B, w.H, w.N, w.P, w.L, w.causal, w.chunk, race.WS_BWD, dev)
    saved = race.alloc_saved(w.B, w.H, w.N, w.P, w.L, w.causal, w.chunk, dev)
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        race.forward(t["Q"], t["K"], t["V"], t["W"], w.P, w.L, w.beta, w.causal, w.chunk, out=O,
                     saved=saved, ws=ws_f)
        race.backward(t["Q"], t["K"], t["V"], t["W"], t["dO"], w.P, w.L, w.beta, w.causal, w.chunk,
                      O=O, saved=saved, ws=ws_b, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps; per-kernel HIP events on the library's stream
    timer = race.StageTimer()
    stage_ms = {}
    stage_n = {}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    with timer:
        for _ in range(args.steps):
            for call in ("fwd", "bwd"):
                if call == "fwd":
                    race.forward(t["Q"], t["K"], t["V"], t["W"], w.P, w.L, w.beta, w.causal, w.chunk,
                                 out=O, saved=saved, ws=ws_f)
                else:
                    race.backward(t["Q"], t["K"], t["V"], t["W"], t["dO"], w.P, w.L, w.beta, w.causal,
                                  w.chunk, O=O, saved=saved, ws=ws_b, grads=grads)
                for name, ms in timer.stages():
                    stage_ms[name] = stage_ms.get(name, 0.0) + ms
                    stage_n[name] = stage_n.get(name, 0) + 1
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.close()
    ms_step = start.elapsed_time(end) / args.steps
    tokens = w.B * w.N
    value = tokens / (ms_step / 1e3)

    layer, kernels = per_token_head_counts(w)
    units = w.token_heads
    # dominant kernel: largest total time in the timed region. A pass runs as
    # one launch per table group, each over every token and its group's
    # features, so one launch's share of the algorithmic count is 1 / launches
    # per step.
    dom = max(stage_ms, key=lambda k: stage_ms[k])
    avg_ms = stage_ms[dom] / stage_n[dom]
    per_step = stage_n[dom] / args.steps
    kb, kf = kernels.get(dom, (0, 0))
    kb, kf = kb / per_step, kf / per_step
    peak_f = MFMA_PEAK[w.dtype]
    t_hbm, t_mma = kb * units / HBM_PEAK, kf * units / peak_f
    if t_hbm >= t_mma:
        roof = {"bound": "hbm", "achieved": kb * units / (avg_ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf * units / (avg_ms / 1e3) / 1e12, "peak": peak_f / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["scope"] = "dominant kernel, one launch (the whole layer step: layer_roofline)"
    roof["traffic"] = measured_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["kernel_avg_ms"] = avg_ms
    roof["launches_per_step"] = per_step
    layer_t = max(layer["bytes"] * units / HBM_PEAK, layer["flops"] * units / peak_f)
    hbm_high_water = torch.cuda.max_memory_allocated() / 2**30
    # the box's own copy bandwidth, beside the nominal peak (outside the timed region)
    copy_gbps = copy_bandwidth(dev)
    mm_tflops = matmul_rate(dev, tdt)
    if roof["unit"] == "GB/s":
        roof["copy_GBps_measured"] = copy_gbps
        roof["frac_of_copy"] = roof["achieved"] / copy_gbps

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "P": w.P, "L": w.L,
                   "chunk": w.chunk, "causal": w.causal, "temperature": w.beta, "seed": w.seed,
                   "qk_dist": w.qk_dist},
        "roofline": roof,
        "layer_roofline": {"bound": "hbm" if layer["bytes"] * units / HBM_PEAK >= layer["flops"] * units / peak_f
                           else "mfma", "frac": layer_t / (ms_step / 1e3),
                           "alg_GBps": layer["bytes"] * units / (ms_step / 1e3) / 1e9,
                           "alg_TFLOPs": layer["flops"] * units / (ms_step / 1e3) / 1e12,
                           "copy_GBps_measured": copy_gbps, "matmul_TFLOPs_measured": mm_tflops,
                           "alg_bytes_per_token_head": layer["bytes"], "alg_flops_per_token_head": layer["flops"]},
        "hbm_peak_GiB": hbm_high_water,
        "hbm_capacity_GiB": torch.cuda.get_device_properties(0).total_memory / 2**30,
        "stages_ms_per_step": {k: v / args.steps for k, v in sorted(stage_ms.items(), key=lambda kv: -kv[1])},
        "wall_s_timed": wall,
    }
    if not args.no_decode:
        out["decode"] = decode_measure(w, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample, w.N))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
