"""Throughput of the MoE layer (moe_forward through the C ABI) on one MI355X.

One step = one moe_forward call over one batch of seeded synthetic input:
router GEMM + top-k, dispatch (counting sort + row gather), grouped gate/up
GEMM with SwiGLU, grouped down GEMM, weighted combine.  Inputs and weights are
resident in HBM before the timed region.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--no-other-configs]

The default workload is the largest single-GPU layer: the DeepSeek-V3-like
layer (T=4096 tokens, hidden 7168, 256 routed experts top-8 + 1 shared
expert, intermediate 2048, e4m3 weights with 128x128 block scales,
activations quantised per token per 128 channels).  The `roofline` object is
for the kernel with the largest share of the step, timed with HIP events
recorded by the library around that kernel's launch on the caller's stream
during the timed steps; `layer_roofline` is the whole step's.  The same line
carries, under `other_configs`, the step time and rooflines of the other four
layer shapes (Tiny, Qwen3-235B-like decode and prefill, Qwen3.5-397B-like),
each timed the same way without a CPU baseline.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec on 1 MI355X + % of HBM / MFMA roofline"


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored), to tell
    whether stored counter data is stale."""
    csrc = os.path.join(ROOT, "expert_ffn_layer_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM traffic of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel") != kernel or d.get("source_hash") != source_hash():
        return None
    return d.get("traffic_bytes")


def cpu_baseline(cfg, li, n_tokens):
    """The oracle, as it stands, on the first n_tokens tokens of the same workload.
    Returns the oracle's result and the timing record."""
    import numpy as np
    import oracle
    from synth import to_numpy_inputs
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in info})) or "?"
    except Exception:  # pragma: no cover
        threads, blas = 1, "?"
    inp = to_numpy_inputs(li)
    n = min(n_tokens, cfg.T)
    inp["x_bf16"] = np.ascontiguousarray(inp["x_bf16"][:n])
    # The same call is repeated until about CPU_MIN_S of work (at most
    # CPU_MAX_REPS calls), so a short sample still gives a steady rate.
    t0 = time.perf_counter()
    ref = oracle.forward(inp)
    reps = 1
    while time.perf_counter() - t0 < CPU_MIN_S and reps < CPU_MAX_REPS:
        oracle.forward(inp)
        reps += 1
    dt = time.perf_counter() - t0
    what = (f"the whole layer ({n} tokens)" if n == cfg.T else f"the first {n} of {cfg.T} tokens")
    return ref, {"value": n * reps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.forward on {what} of {cfg.name} (seed {cfg.seed}, same inputs as the "
                      f"GPU steps), {reps} call(s) in {dt:.2f} s, fp32 NumPy; BLAS {blas} with "
                      f"{threads} threads; {len(os.sched_getaffinity(0))} cores in this process's "
                      f"affinity, os.cpu_count()={os.cpu_count()}"}


def device_info(dev):
    """The GPU the run used (name, compute units, memory) and a plain 1 GiB
    device-to-device copy's rate, as context for the HBM fractions."""
    import torch
    pr = torch.cuda.get_device_properties(dev)
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9   # read + write bytes
    del a, b
    torch.cuda.empty_cache()
    return {"name": pr.name, "gcn_arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count, "hbm_gib": round(pr.total_memory / 2 ** 30, 1),
            "copy_1gib_gbs": round(gbs, 1)}


def routing_stats(counts):
    """Load balance of the routed experts held here: how many got no row or one
    row, the largest group, and the spread of group sizes (std / mean)."""
    import numpy as np
    c = np.asarray(counts, dtype=np.float64)
    mean = c.mean() if c.size else 0.0
    return {"empty_experts": int((c == 0).sum()), "one_row_experts": int((c == 1).sum()),
            "max_group_rows": int(c.max()) if c.size else 0,
            "load_std_over_mean": round(float(c.std() / mean), 4) if mean > 0 else None}


def sampled_parity(out, idx, ref):
    """The timed steps' output on the oracle's tokens (the whole layer by
    default) against the oracle (its own router logits, so a near-tie may pick
    another expert: such tokens are counted, not compared)."""
    import numpy as np
    import torch
    n = ref.out.shape[0]
    u = out[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    gpu = (u.astype(np.uint32) << 16).view(np.float32)
    same = (idx[:n].cpu().numpy() == ref.topk_idx).all(axis=1)
    if not same.any():
        return {"tokens": n, "routing_differs": int(n), "max_token_rel_err": None}
    num = np.abs(gpu - ref.out).max(axis=1)
    den = np.maximum(np.abs(ref.out).max(axis=1), 1e-30)
    return {"tokens": n, "routing_differs": int((~same).sum()),
            "max_token_rel_err": float((num / den)[same].max())}


CPU_MIN_S, CPU_MAX_REPS = 10.0, 16     # oracle timing: >= ~10 s of CPU work, bounded
# Tokens the oracle runs on for each workload's CPU baseline: the whole layer
# (every token) where one oracle call takes well under a minute on the host.
CPU_TOKENS = {"tiny": 64, "qwen3_235b_decode": 64, "qwen3_235b_prefill": 8192,
              "qwen35_397b_zipf": 1024, "deepseek_v3_fp8": 4096,
              "qwen3_235b_decode_mxfp8": 64, "qwen3_235b_prefill_mxfp8": 8192,
              "qwen3_235b_decode_ep8": 64, "qwen3_235b_prefill_ep4": 8192,
              "deepseek_v3_decode_ep16": 64, "qwen3_235b_decode_mxfp8_ep8": 64}
DEFAULT_CONFIG = "deepseek_v3_fp8"
OTHER_CONFIGS = ("tiny", "qwen3_235b_decode", "qwen3_235b_prefill", "qwen35_397b_zipf")


def measure(cfg, steps, warmup, graph_probe=False):
    """Time `steps` moe_forward calls of one workload after `warmup` untimed ones.

    Returns the record fields (timing, rooflines, per-kernel times) and the
    device buffers the last step wrote (out, idx) plus the generated inputs."""
    import numpy as np
    import torch

    import expert_ffn_layer_gemm_amd as moe
    from expert_ffn_layer_gemm_amd import accounting as acc
    from synth import generate_layer

    dev = torch.device("cuda:0")
    li = generate_layer(cfg, dev)
    shape = moe.shape_of(cfg)
    ws = torch.empty(moe.moe_forward_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_forward(shape, li.x, li.w_router, li.router_bias, li.w_gate, li.w_up, li.w_down,
                        li.s_gate, li.s_up, li.s_down, out, idx, w, ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # One untimed step with events around every launch: find the dominant kernel
    # (in this mode the library runs its two FFN kernel chains one after the
    # other, so each launch is timed alone).
    moe.moe_profile_start(1, 0, 64)
    step()
    launches = [moe.moe_profile_read(i) for i in range(moe.moe_profile_count())]
    moe.moe_profile_stop()
    dom = int(np.argmax([ms for ms, _ in launches]))
    dom_name = launches[dom][1]

    # Timed region: K steps; the library records one event pair around the
    # dominant kernel's launch in each step.
    moe.moe_profile_start(2, dom, steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    kern_ms = [moe.moe_profile_read(i)[0] for i in range(moe.moe_profile_count())]
    moe.moe_profile_stop()
    ms_per_step = total_ms / steps
    value = cfg.T * steps / (total_ms / 1e3)

    # After the timed region: the spread of single steps (an event pair
    # around each of K more steps).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    one = np.array([a.elapsed_time(b) for a, b in evs])
    spread = {"median_ms": float(np.median(one)), "p90_ms": float(np.percentile(one, 90)),
              "min_ms": float(one.min()), "steps": int(len(one))}

    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.E)
    counts = counts[cfg.e_first:cfg.e_first + cfg.E_loc]      # the experts held here
    if cfg.n_shared:
        counts = np.concatenate([counts, [cfg.T] * cfg.n_shared])
    dtype = cfg.wdtype if cfg.wdtype in ("fp8", "mxfp8") else "bf16"
    kern_s = float(np.mean(kern_ms)) / 1e3
    if dom_name.startswith(("skinny_", "tiled_")):
        work = acc.kernel_work(dom_name, counts, cfg.H, cfg.I, cfg.wdtype, acc.skinny_max_rows(cfg.T))
    else:
        work = None
    roof = acc.roofline(work, kern_s, dtype) if work else None
    if roof is not None:
        roof.update({"kernel": dom_name, "kernel_ms": kern_s * 1e3,
                     "algorithmic_bytes": work.bytes, "algorithmic_flops": work.flops,
                     "traffic": stored_traffic(cfg.name, dom_name)})
    # Roofline of every grouped-FFN launch of the untimed profiling step.
    kernel_roofs = {}
    for i, (ms, n) in enumerate(launches):
        if n.startswith(("skinny_", "tiled_")):
            wk = acc.kernel_work(n, counts, cfg.H, cfg.I, cfg.wdtype, acc.skinny_max_rows(cfg.T))
            if wk.groups:
                rf = acc.roofline(wk, ms / 1e3, dtype)
                kernel_roofs[f"{i}:{n}"] = {"ms": round(ms, 4), "groups": wk.groups,
                                            "bound": rf["bound"], "frac": round(rf["frac"], 4)}
    layer = acc.layer_work(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.wdtype, counts)
    layer_roof = acc.roofline(layer, ms_per_step / 1e3, dtype)

    graph = None
    if graph_probe:
        # The same step captured once on a side stream and replayed K times.
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            moe.moe_forward(shape, li.x, li.w_router, li.router_bias, li.w_gate, li.w_up,
                            li.w_down, li.s_gate, li.s_up, li.s_down, out, idx, w, ws,
                            stream=torch.cuda.current_stream())
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph = {"ms_per_step": g0.elapsed_time(g1) / steps}

    config = {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
              "I": cfg.I, "n_shared": cfg.n_shared, "weights": cfg.wdtype,
              **({"expert_share": [cfg.e_first, cfg.e_first + cfg.E_loc]} if cfg.e_local else {}),
              "touched_experts": int(layer.groups),
              **routing_stats(counts[:cfg.E_loc])}
    rec = {"value": value, "ms_per_step": ms_per_step, "dtype": dtype, "config": config,
           "roofline": roof, "layer_roofline": layer_roof,
           "per_kernel_ms": {f"{i}:{n}": round(ms, 4) for i, (ms, n) in enumerate(launches)},
           "grouped_ffn_rooflines": kernel_roofs, "wall_s_timed_region": t_wall,
           "single_steps": spread, "graph_replay": graph}
    return rec, li, out, idx


def summary(rec):
    """The short form of a workload's record carried under other_configs."""
    r, lr = rec["roofline"], rec["layer_roofline"]
    return {"tokens_per_s": rec["value"], "ms_per_step": rec["ms_per_step"], "dtype": rec["dtype"],
            "layer_roofline": {k: lr[k] for k in ("bound", "achieved", "unit", "frac")},
            "dominant_kernel": None if r is None else
            {"kernel": r["kernel"], "kernel_ms": r["kernel_ms"], "bound": r["bound"], "frac": r["frac"]},
            "touched_experts": rec["config"]["touched_experts"],
            "max_group_rows": rec["config"]["max_group_rows"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only --config (no other_configs records)")
    ap.add_argument("--cpu-tokens", type=int, default=None)
    ap.add_argument("--graph-probe", action="store_true",
                    help="also time K replays of moe_forward captured in a HIP graph (extra field)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the MoE layer on one MI355X; "
              "runs on more than one GPU are not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import config_by_name

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": 1 << 30, "launches": 3}))
        return

    cfg = config_by_name(args.config)
    print(f"bench: timing {cfg.name}", file=sys.stderr, flush=True)
    rec, li, out, idx = measure(cfg, args.steps, args.warmup, args.graph_probe)
    device = device_info(dev)

    cpu = parity = None
    if not args.no_cpu_baseline:
        print(f"bench: oracle on the host for {cfg.name}", file=sys.stderr, flush=True)
        ref, cpu = cpu_baseline(cfg, li, args.cpu_tokens or CPU_TOKENS.get(cfg.name, 64))
        parity = sampled_parity(out, idx, ref)
        del ref
    del li, out, idx
    torch.cuda.empty_cache()

    others = None
    if not args.no_other_configs and args.config == DEFAULT_CONFIG:
        others = {}
        for name in OTHER_CONFIGS:
            print(f"bench: timing {name}", file=sys.stderr, flush=True)
            r, *_ = measure(config_by_name(name), args.steps, args.warmup)
            others[name] = summary(r)
            torch.cuda.empty_cache()

    res = {
        "metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "layer_roofline": rec["layer_roofline"],
        "per_kernel_ms": rec["per_kernel_ms"],
        "grouped_ffn_rooflines": rec["grouped_ffn_rooflines"],
        "wall_s_timed_region": rec["wall_s_timed_region"],
        "single_steps": rec["single_steps"],
        "device": device,
        "graph_replay": rec["graph_replay"],
        "cpu_baseline": cpu,
        "parity": parity,
        "other_configs": others,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
