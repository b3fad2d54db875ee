"""Throughput of the MI355X MoE layer forward (router -> dispatch -> grouped
SwiGLU experts -> combine) on a seeded synthetic Qwen-MoE-shaped layer.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one whole ``moe_forward`` over the batch
(all stages, inputs already resident in HBM).  ``value`` is tokens/s.  Two
timed regions run back to back: a clean one for ``value`` and one with HIP
events bracketing every library kernel (recorded on the stream each kernel is
launched on) for the per-kernel durations and the roofline of the dominant
kernel.  The float64 oracle is timed on a bounded token sample on the host
cores as ``cpu_baseline`` (a reported baseline only).
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

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "MoE-layer tokens/sec at Qwen3-30B-A3B shape; grouped-GEMM % bf16 peak"
DEFAULT_WORKLOAD = "qwen3_30b_a3b_prefill"

# MI355X published peaks (dense)
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def y_bytes_per_value(cfg):
    """Bytes per packed expert output value as the layer forward stores them:
    bf16 layers whose down projection runs on a 256-row kernel (at least 96
    rows per expert on average) keep fp16 values plus one int32 exponent per
    64 columns; otherwise fp32."""
    P = cfg.num_tokens * cfg.top_k
    groups = min(cfg.num_experts, P)
    avg = (P + groups - 1) // groups
    if cfg.dtype == "bf16" and avg >= 96 and cfg.hidden_size % 64 == 0:
        return 2.0 + 4.0 / 64
    return 4.0


def kernel_work(name, cfg, touched, touched_shared=True):
    """Algorithmic FLOPs and HBM bytes of ONE launch of a library kernel.

    Bytes count each tensor the kernel must move once: weights of touched
    experts only, activations read/written once; tile padding and re-reads are
    not counted."""
    T, H, E, k, I = cfg.num_tokens, cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.intermediate_size
    Is = cfg.shared_intermediate_size
    P = T * k
    es = 2 if cfg.dtype == "bf16" else 4  # activations, weights and h
    ys = y_bytes_per_value(cfg)  # routed y; the shared expert's output is fp32
    if name in ("ffn_gate_up_bf16", "ffn_gate_up_f32"):
        # weights of touched experts, every token row once, h written once
        return 4.0 * P * H * I, touched * 2 * I * H * es + T * H * es + P * I * es
    if name in ("ffn_down_bf16", "ffn_down_f32"):
        return 2.0 * P * H * I, touched * H * I * es + P * I * es + P * H * ys
    if name == "shared_gate_up_bf16":
        return 4.0 * T * H * Is, 2 * Is * H * es + T * H * es + T * Is * es
    if name == "shared_down_bf16":
        return 2.0 * T * H * Is, H * Is * es + T * Is * es + T * H * 4
    if name in ("router_logits_bf16", "router_logits_f32"):
        C = E + (1 if Is else 0)
        return 2.0 * T * H * C, T * H * es + C * H * es + T * C * 4
    if name == "router_topk":
        return 0.0, T * E * 4 + 2 * P * 4
    if name == "router_topk_hist":
        # logits read, ids and weights written, the per-segment histogram written
        U = (P + 127) // 128
        return 0.0, T * E * 4 + 2 * P * 4 + U * E * 4
    if name == "topk_dispatch_small":
        return 0.0, T * E * 4 + 2 * P * 4 + 3 * P * 4 + (2 * E + 1) * 4
    if name == "dispatch_hist":
        return 0.0, P * 4
    if name == "dispatch_scan":
        return 0.0, 2 * E * 4
    if name == "dispatch_scatter":
        return 0.0, P * 4 + 3 * P * 4
    if name == "combine":
        # y and the shared output (fp32) read once, fp32 output written once
        return 0.0, P * H * ys + P * 8 + T * H * 4 + (T * H * 4 if Is else 0)
    return 0.0, 0.0


# rocprofv3 counter summaries: profiles/<kernel>_<workload>_traffic.txt holds
# "key: value" lines, among them the SHA-256 of the kernel's source file at the
# time the counters were taken.
KERNEL_SOURCES = {
    "ffn_gate_up_bf16": "route_dispatch_grouped_amd/csrc/grouped_gemm_bf16.hip",
    "ffn_down_bf16": "route_dispatch_grouped_amd/csrc/grouped_gemm_bf16.hip",
    "combine": "route_dispatch_grouped_amd/csrc/combine.hip",
    "router_topk_hist": "route_dispatch_grouped_amd/csrc/dispatch.hip",
    "dispatch_scan": "route_dispatch_grouped_amd/csrc/dispatch.hip",
    "dispatch_scatter": "route_dispatch_grouped_amd/csrc/dispatch.hip",
}


def measured_traffic(name, workload):
    """HBM bytes per launch of kernel `name` from its committed FETCH_SIZE and
    WRITE_SIZE summary, each scaled by what the counter read for a plain device
    copy of known size; None when there is no summary or the kernel's source
    has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_{workload}_traffic.txt")
    src = KERNEL_SOURCES.get(name)
    if src is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    with open(os.path.join(ROOT, src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if kv.get("source_sha256") != sha:
        return None
    try:
        copy_bytes = float(kv["copy_bytes"])
        fetch_scale = copy_bytes / (float(kv["copy_fetch_kib"]) * 1024.0)
        write_scale = copy_bytes / (float(kv["copy_write_kib"]) * 1024.0)
        return (float(kv["fetch_kib_per_launch"]) * 1024.0 * fetch_scale +
                float(kv["write_kib_per_launch"]) * 1024.0 * write_scale)
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def roofline_entry(name, cfg, avg_s, touched):
    flops, nbytes = kernel_work(name, cfg, touched)
    peak_f = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    t_f = flops / (peak_f * 1e12)
    t_b = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_f >= t_b and flops > 0:
        ach = flops / avg_s / 1e12
        return {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": round(ach, 2), "peak": peak_f,
                "unit": "TFLOP/s", "frac": round(ach / peak_f, 4), "traffic": None,
                "kernel": name, "avg_us": round(avg_s * 1e6, 2), "algorithmic_flops": flops,
                "algorithmic_bytes": nbytes}
    ach = nbytes / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": name,
            "avg_us": round(avg_s * 1e6, 2), "algorithmic_flops": flops, "algorithmic_bytes": nbytes}


def host_info():
    """The host CPU model, the threads available to this process, and the BLAS
    library NumPy runs on with its thread count."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                blas = f"{d.get('internal_api')} {d.get('version')} ({os.path.basename(d.get('filepath', ''))})"
                threads = int(d.get("num_threads", 1))
                break
    except Exception:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "affinity_cpus": affinity, "blas": blas,
            "blas_threads": threads if threads is not None else affinity}


def cpu_baseline(cfg, inp, sample_tokens, target_s, repeats=3):
    """Time the float64 oracle on the first `sample_tokens` tokens of the
    workload (grown toward `target_s` seconds per run, at most the whole
    batch); the median of `repeats` runs."""
    import oracle
    info = host_info()
    S = min(sample_tokens, cfg.num_tokens)
    sub = dict(inp)

    def run(n):
        sub["x"] = inp["x"][:n]
        t0 = time.perf_counter()
        oracle.forward(sub, cfg.top_k, cfg.renormalize)
        return time.perf_counter() - t0

    dt = run(S)
    # grow the sample once if it was far below the target duration
    if dt < target_s / 3 and S < cfg.num_tokens:
        S2 = min(cfg.num_tokens, int(S * min(8.0, target_s / max(dt, 1e-3))))
        if S2 > S:
            S = S2
            dt = run(S)
    times = [dt] + [run(S) for _ in range(repeats - 1)]
    med = float(np.median(times))
    return {"value": round(S / med, 2), "unit": "tokens/s", "cores": int(info["blas_threads"]), "kind": "oracle",
            "sample": f"float64 NumPy oracle forward (router, top-k, dispatch plan, per-expert SwiGLU, combine) "
                      f"over the first {S} of {cfg.num_tokens} tokens with the full layer weights; median of "
                      f"{len(times)} runs {med:.2f} s",
            "seconds": round(med, 3), "runs_s": [round(t, 3) for t in times], **info}


def y_storage(cfg):
    """How the forward stores the packed expert outputs y, i.e. the byte basis
    of the down projection's and the combine's algorithmic bytes."""
    b = y_bytes_per_value(cfg)
    fmt = ("fp16 values scaled by a power of two, one int32 exponent per (row, 64 columns)" if b < 4
           else "fp32")
    return {"bytes_per_value": b, "format": fmt,
            "note": "down and combine algorithmic bytes count y at bytes_per_value; at fp32 y (4 B/value) they "
                    "would count P*H*(4 - bytes_per_value) more bytes each"}


SECONDARY_WORKLOAD = "qwen15_moe_decode"
SETTLE_FORWARDS = 120  # forwards after which the layer runs at its steady clock (see "steady state" in main)


def _percentiles(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"p10_ms": round(float(np.percentile(a, 10)), 4), "p50_ms": round(float(np.percentile(a, 50)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "mean_ms": round(float(a.mean()), 4)}


def timed_forwards(torch, fwd, steps, flush=None):
    """Per-forward durations (ms) from HIP events on the current stream, which
    the forward joins back to (its shared expert's stream included).  With
    `flush`, a scratch stream of memory runs before every forward, outside
    the events, so each forward starts with cold caches (L2 and the MALL)."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(st)
        fwd()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def decode_measure(rdg, torch, seed, steps=400, warmup=50, flushed_steps=100, flush_mib=1024):
    """The memory-bound decode shape beside the headline: one forward per
    step, reported as tokens/s and as weight bytes streamed per second against
    the HBM peak.  Bytes per step: the touched experts' w13 and w2, the shared
    expert's weights, the router and gate rows (activations are negligible).
    Three regimes, each with event-timed p10/p50/p90: back-to-back forwards
    (weights may stay in the 256 MB MALL between steps); forwards each
    preceded by a read-only pass over `flush_mib` MiB (a sum), which leaves
    the L2s and the MALL holding clean lines of that buffer and none of the
    weights; and forwards each preceded by a copy of `flush_mib` MiB, whose
    writes leave the caches full of dirty lines that are written back to HBM
    while the forward runs."""
    cfg = workloads.config(SECONDARY_WORKLOAD)
    inp = workloads.generate(cfg, seed=seed)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = {kk: dev(v) for kk, v in inp.items()}
    layer = rdg.MoeLayer(d["router_weight"], d["w13"], d["w2"], cfg.top_k, router_bias=d.get("router_bias"),
                         shared_w13=d.get("shared_w13"), shared_w2=d.get("shared_w2"),
                         shared_gate=d.get("shared_gate"), renormalize=cfg.renormalize)
    x = d["x"]
    layer.reserve(cfg.num_tokens, x.device)
    for _ in range(warmup):
        layer(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    warm = timed_forwards(torch, lambda: layer(x), steps)
    n = flush_mib * (1 << 20) // 4
    fa = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    fb = torch.empty_like(fa)
    cold = timed_forwards(torch, lambda: layer(x), flushed_steps, flush=lambda: torch.sum(fa))
    dirty = timed_forwards(torch, lambda: layer(x), flushed_steps, flush=lambda: fb.copy_(fa))
    del fa, fb
    r = rdg.moe_router_topk(x, d["router_weight"], cfg.top_k, renormalize=cfg.renormalize)
    counts = rdg.moe_dispatch_plan(r["topk_ids"], None, cfg.num_experts)["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    H, I, Is, E = cfg.hidden_size, cfg.intermediate_size, cfg.shared_intermediate_size, cfg.num_experts
    nbytes = touched * 3 * I * H * 2 + 3 * Is * H * 2 + (E + 1) * H * 2
    gbs = nbytes / dt / 1e9

    def regime(ms, label):
        p = _percentiles(ms)
        gb = {f"gbs_{q}": round(nbytes / (p[f"{q}_ms"] * 1e-3) / 1e9, 1) for q in ("p10", "p50", "p90")}
        return {"caches": label, "forwards": len(ms), **p, **gb,
                "frac_hbm_peak_p50": round(gb["gbs_p50"] / PEAK_HBM_GBS, 4)}

    res = {"workload": cfg.name, "steps": steps, "warmup": warmup, "ms_per_step": round(dt * 1e3, 4),
           "value": round(cfg.num_tokens / dt, 1), "unit": "tokens/s", "experts_touched": touched,
           "weight_bytes_per_step": nbytes, "achieved": round(gbs, 1), "achieved_unit": "GB/s",
           "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "unflushed": regime(warm, "back-to-back forwards (weights may stay in the MALL)"),
           "flushed": regime(cold, f"a read-only pass over {flush_mib} MiB before every forward (cold L2 and "
                                   "MALL)"),
           "flushed_dirty": regime(dirty, f"a {flush_mib} MiB device copy before every forward (cold L2 and MALL, "
                                          "their dirty lines written back during the forward)")}
    # one rank of an 8-way tensor-parallel split (I / 8 and Is / 8, router and
    # gate replicated): the same tokens stream an eighth of the expert weights
    G = 8
    if I % (16 * G) == 0 and Is % (16 * G) == 0:
        w13, w2 = rdg.moe_tp_slice_experts(d["w13"], d["w2"], G, 0)
        s13, s2 = rdg.moe_tp_slice_experts(d["shared_w13"], d["shared_w2"], G, 0)
        rank = rdg.MoeLayer(d["router_weight"], w13, w2, cfg.top_k, router_bias=d.get("router_bias"),
                            shared_w13=s13, shared_w2=s2, shared_gate=d.get("shared_gate"),
                            renormalize=cfg.renormalize)
        rank.reserve(cfg.num_tokens, x.device)
        for _ in range(warmup):
            rank(x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            rank(x)
        torch.cuda.synchronize()
        dtr = (time.perf_counter() - t0) / steps
        nb = (touched * 3 * I * H * 2 + 3 * Is * H * 2) // G + (E + 1) * H * 2
        res["tp8_rank"] = {"intermediate_size": I // G, "shared_intermediate_size": Is // G,
                           "ms_per_step": round(dtr * 1e3, 4), "weight_bytes_per_step": nb,
                           "achieved": round(nb / dtr / 1e9, 1), "achieved_unit": "GB/s"}
    return res


def tp_measure(rdg, torch, cfg, d, steps, warmup=10, sizes=(2, 4, 8)):
    """One tensor-parallel rank's layer at the headline shape: the experts'
    intermediate size split over tp ranks (weights sliced from the full ones
    by moe_tp_load_expert), router replicated.  Per rank: ms per forward and
    the grouped FFN's fraction of the bf16 peak (its flops are 1/tp of the
    full layer's).  The cross-rank sum of the outputs is not part of it."""
    res = []
    for tp in sizes:
        if cfg.intermediate_size % tp:
            continue
        w13, w2 = rdg.moe_tp_slice_experts(d["w13"], d["w2"], tp, 0)
        layer = rdg.MoeLayer(d["router_weight"], w13, w2, cfg.top_k, router_bias=d.get("router_bias"),
                             renormalize=cfg.renormalize)
        x = d["x"]
        layer.reserve(cfg.num_tokens, x.device)
        for _ in range(warmup):
            layer(x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer(x)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        rdg.profile_enable(True)
        for _ in range(steps):
            layer(x)
        torch.cuda.synchronize()
        rdg.profile_enable(False)
        k = rdg.profile_collect()
        Ip = cfg.intermediate_size // tp
        ent = {"tp": tp, "intermediate_size": Ip, "ms_per_step": round(dt * 1e3, 4),
               "value": round(cfg.num_tokens / dt, 1), "unit": "tokens/s",
               "kernels_us": {n: round(ms / c * 1e3, 2) for n, (ms, c) in k.items()}}
        if "ffn_gate_up_bf16" in k and "ffn_down_bf16" in k:
            t_ffn = sum(k[n][0] / k[n][1] for n in ("ffn_gate_up_bf16", "ffn_down_bf16")) / 1e3
            fl = 6.0 * cfg.num_tokens * cfg.top_k * cfg.hidden_size * Ip
            ent["grouped_ffn"] = {"tflops": round(fl / t_ffn / 1e12, 2),
                                  "frac_bf16_peak": round(fl / t_ffn / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "us": round(t_ffn * 1e6, 2)}
        res.append(ent)
        log(f"[bench] tp{tp} rank layer (I={Ip}): {ent['ms_per_step']} ms/step, "
            f"ffn {ent.get('grouped_ffn')}")
        del layer, w13, w2
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps; the clocks settle after about 15 forwards of this size")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(workloads.CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--cpu-target-seconds", type=float, default=15.0)
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event region")
    ap.add_argument("--no-secondary", action="store_true",
                    help=f"skip the {SECONDARY_WORKLOAD} measurement reported beside the headline workload")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the steps, run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the MoE layer forward runs on a single GPU "
                                   "and has no multi-GPU path (its expert- and tensor-parallel pieces are "
                                   "single-GPU building blocks, with no collectives); run with --gpus 1"}))
        sys.exit(2)

    import torch

    import route_dispatch_grouped_amd as rdg

    if not os.path.exists(rdg.LIB_PATH):  # a fresh checkout: build once, otherwise load what is built
        from route_dispatch_grouped_amd.build import build
        build()

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = workloads.config(args.workload)
    log(f"[bench] generating {cfg.name} (seed {args.seed})")
    t0 = time.perf_counter()
    inp = workloads.generate(cfg, seed=args.seed)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = {kk: dev(v) for kk, v in inp.items()}
    layer = rdg.MoeLayer(d["router_weight"], d["w13"], d["w2"], cfg.top_k, router_bias=d.get("router_bias"),
                         shared_w13=d.get("shared_w13"), shared_w2=d.get("shared_w2"),
                         shared_gate=d.get("shared_gate"), renormalize=cfg.renormalize)
    x = d["x"]
    layer.reserve(cfg.num_tokens, x.device)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer(x)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # ---- timed region A: value
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        layer(x)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = cfg.num_tokens * args.steps / wall
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (events {ev_ms / args.steps:.3f} ms)")

    # ---- steady state.  A process's first forwards run inside a transient of
    # the GPU's power management: right after the first (code loading) one
    # fast forward, then up to ~35 % slower ones that settle over ~40
    # forwards (prefill shape).  With few warm-up forwards region A falls in
    # it, so the same K forwards are timed again once the process has run
    # at least SETTLE_FORWARDS of them; the per-kernel region below follows.
    steady = None
    if not args.no_profile:
        extra = max(0, SETTLE_FORWARDS - args.warmup - args.steps)
        for _ in range(extra):
            layer(x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer(x)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        steady = {"forwards_before": args.warmup + args.steps + extra, "steps": args.steps,
                  "ms_per_step": round(wall_s * 1e3 / args.steps, 4),
                  "value": round(cfg.num_tokens * args.steps / wall_s, 1), "unit": "tokens/s"}
        log(f"[bench] steady state after {steady['forwards_before']} forwards: {steady['ms_per_step']} ms/step")

    # routing statistics of this batch (outside the timed regions)
    r = rdg.moe_router_topk(x, d["router_weight"], cfg.top_k, router_bias=d.get("router_bias"),
                            renormalize=cfg.renormalize)
    plan = rdg.moe_dispatch_plan(r["topk_ids"], None, cfg.num_experts)
    counts = plan["counts"].cpu().numpy()
    touched = int((counts > 0).sum())

    # ---- timed region B: per-kernel HIP events
    kernels = {}
    if not args.no_profile:
        rdg.profile_enable(True)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            layer(x)
        torch.cuda.synchronize()
        rdg.profile_enable(False)
        kernels = rdg.profile_collect()
        log("[bench] per-kernel: " + ", ".join(f"{n} {ms / c * 1e3:.1f}us" for n, (ms, c) in kernels.items()))

    # expert-parallel routing table of this batch's routing, as rank 2 of 8
    # (experts [E/4, 3E/8)): outside the layer step, timed on its own
    ep = None
    if not args.no_profile:
        E = cfg.num_experts
        lo, hi = E * 2 // 8, E * 3 // 8
        ids_flat, w_flat = r["topk_ids"].reshape(-1), r["topk_weights"].reshape(-1)
        for _ in range(3):
            rdg.moe_ep_routing_table(ids_flat, w_flat, cfg.num_tokens, cfg.top_k, lo, hi, trim=False)
        torch.cuda.synchronize()
        rdg.profile_enable(True)
        for _ in range(args.steps):
            rdg.moe_ep_routing_table(ids_flat, w_flat, cfg.num_tokens, cfg.top_k, lo, hi, trim=False)
        torch.cuda.synchronize()
        rdg.profile_enable(False)
        ms, c = rdg.profile_collect()["ep_routing_table"]
        P = cfg.num_tokens * cfg.top_k
        nbytes = P * 8 + P * 12 + 8  # ids + weights read; (token, expert, weight) written; counts
        avg_s = ms / c / 1e3
        ep = {"avg_us": round(avg_s * 1e6, 2), "local_range": [lo, hi], "algorithmic_bytes": nbytes,
              "achieved": round(nbytes / avg_s / 1e9, 1), "unit": "GB/s",
              "frac": round(nbytes / avg_s / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] ep routing table: {ep['avg_us']} us ({ep['achieved']} GB/s)")

    # group-limited top-k on this batch (experts in 8 groups, 4 kept): the
    # selection kernel alone, timed like the plain one (outside the layer step)
    grouped = None
    if not args.no_profile and cfg.num_experts % 8 == 0 and cfg.top_k <= 4 * (cfg.num_experts // 8):
        ng, tg = 8, 4
        for _ in range(3):
            rdg.moe_router_topk_grouped(x, d["router_weight"], cfg.top_k, ng, tg, router_bias=d.get("router_bias"),
                                        renormalize=cfg.renormalize)
        torch.cuda.synchronize()
        rdg.profile_enable(True)
        for _ in range(args.steps):
            rdg.moe_router_topk_grouped(x, d["router_weight"], cfg.top_k, ng, tg, router_bias=d.get("router_bias"),
                                        renormalize=cfg.renormalize)
        torch.cuda.synchronize()
        rdg.profile_enable(False)
        prof = rdg.profile_collect()
        ms, c = prof["router_topk_grouped"]
        avg_s = ms / c / 1e3
        nbytes = cfg.num_tokens * cfg.num_experts * 4 + 2 * cfg.num_tokens * cfg.top_k * 4
        grouped = {"avg_us": round(avg_s * 1e6, 2), "n_group": ng, "topk_group": tg, "algorithmic_bytes": nbytes,
                   "achieved": round(nbytes / avg_s / 1e9, 1), "unit": "GB/s",
                   "frac": round(nbytes / avg_s / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] grouped top-k ({ng} groups, {tg} kept): {grouped['avg_us']} us")

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per_kernel = {}
    roof = None
    dominant = None
    for n, (ms, c) in kernels.items():
        avg_s = ms / c / 1e3
        ent = roofline_entry(n, cfg, avg_s, touched)
        per_kernel[n] = {"avg_us": round(avg_s * 1e6, 2), "launches_per_step": c // max(args.steps, 1),
                         "bound": ent["bound"], "achieved": ent["achieved"], "unit": ent["unit"],
                         "frac": ent["frac"]}
        tr = measured_traffic(n, cfg.name)
        if tr is not None:
            # HBM bytes from the committed FETCH_SIZE/WRITE_SIZE summary over this run's duration
            per_kernel[n]["hbm_traffic_bytes"] = round(tr)
            per_kernel[n]["hbm_gbs_counters"] = round(tr / avg_s / 1e9, 1)
            per_kernel[n]["hbm_frac_counters"] = round(tr / avg_s / 1e9 / PEAK_HBM_GBS, 4)
        if dominant is None or ms > kernels[dominant][0]:
            dominant = n
    if dominant is not None:
        ms, c = kernels[dominant]
        roof = roofline_entry(dominant, cfg, ms / c / 1e3, touched)
        tr = measured_traffic(dominant, cfg.name)
        roof["traffic"] = None if tr is None else round(tr)

    # grouped FFN (gate/up + down) as a fraction of bf16 peak
    ffn = None
    if "ffn_gate_up_bf16" in kernels and "ffn_down_bf16" in kernels:
        t_ffn = sum(kernels[n][0] / kernels[n][1] for n in ("ffn_gate_up_bf16", "ffn_down_bf16")) / 1e3
        fl = 6.0 * cfg.num_tokens * cfg.top_k * cfg.hidden_size * cfg.intermediate_size
        ffn = {"tflops": round(fl / t_ffn / 1e12, 2), "frac_bf16_peak": round(fl / t_ffn / 1e12 / PEAK_BF16_TFLOPS, 4),
               "us": round(t_ffn * 1e6, 2)}

    secondary = None
    if not args.no_secondary and cfg.name == DEFAULT_WORKLOAD:
        log(f"[bench] secondary: {SECONDARY_WORKLOAD}")
        secondary = decode_measure(rdg, torch, args.seed)
        log(f"[bench] {SECONDARY_WORKLOAD}: {secondary['ms_per_step']} ms/step, {secondary['achieved']} GB/s "
            f"({100 * secondary['frac_hbm_peak']:.1f} % of HBM peak); p50 unflushed "
            f"{secondary['unflushed']['p50_ms']} ms ({secondary['unflushed']['gbs_p50']} GB/s), flushed "
            f"{secondary['flushed']['p50_ms']} ms ({secondary['flushed']['gbs_p50']} GB/s)")

    tp = None
    if not args.no_secondary and cfg.name == DEFAULT_WORKLOAD and cfg.dtype == "bf16":
        tp = tp_measure(rdg, torch, cfg, d, args.steps)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(cfg, inp, args.cpu_sample_tokens, args.cpu_target_seconds)
        log(f"[bench] oracle: {cpu['value']} tokens/s ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_tokens": cfg.num_tokens, "hidden_size": cfg.hidden_size,
                   "num_experts": cfg.num_experts, "top_k": cfg.top_k, "intermediate_size": cfg.intermediate_size,
                   "shared_intermediate_size": cfg.shared_intermediate_size, "renormalize": cfg.renormalize,
                   "seed": args.seed, "experts_touched": touched, "max_expert_rows": int(counts.max()),
                   "inputs": "x~N(0,1), weights~N(0,0.02), bf16 RNE; seeded PCG64 streams"},
        "roofline": roof,
        "steady_state": steady,
        "y_storage": y_storage(cfg),
        "grouped_ffn": ffn,
        "kernels": per_kernel,
        "ep_routing_table": ep,
        "router_topk_grouped": grouped,
        "decode": secondary,
        "tp_sliced": tp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
