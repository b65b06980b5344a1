"""Benchmark of the NVFP4 fused-MoE layer on one MI355X.

One step = one forward of the whole layer (per-token quantize, router top-k,
expandInputRows permutation, GEMM1 + SwiGLU, re-quantization + GEMM2,
finalize) over one batch of seeded synthetic tokens already resident in HBM.
Default run: the decode-shaped layer (T=64, H=2048, E=128, top-8, I=768) is
the headline line, and a `configs` list in the same JSON line times every
other configuration the same way in the same run: the tiny layer (T=16), the
prefill-shaped layer (T=4096, Zipf-skewed routing; MFMA roofline), the
quantize-only workload (per-token NVFP4 quantization of x bf16 [16384, 7168];
one step = one launch, HBM roofline) and the large layer (H=7168, E=256,
I=2048) at T = 1, 7 and 2048, each with its own roofline and CPU-oracle
baseline.  `--layer N [--T T]` times one workload alone.  Prints one JSON
line.

Timing: `steps` forwards after `warmup` untimed ones, bracketed by
synchronizations; wall time gives `value` (tokens/s).  By default the timed
forwards are captured into one HIP graph and replayed once (a decode
deployment replays one graph per model step holding every layer; `--eager`
launches the kernels directly).  After the graph replay the same forwards
are timed a second time, launched directly, each recording HIP events
around its four kernels on its own stream (`eager_ms_per_step`, reported
beside `ms_per_step`): those intervals give each kernel's mean duration, and
the dominant kernel's algorithmic bytes (or FLOPs) over that duration is
`roofline.achieved`.  (A HIP graph's event-record nodes leave the events'
timestamps as their last eager record had them, so the graph replay itself
cannot time its kernels.)  Expert weights rotate over `--rotate` copies so
consecutive steps do not find them in the 256 MB Infinity Cache.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_sources_digest():
    """sha256 over the HIP/C++ sources of the library (names and contents)."""
    import hashlib

    d = hashlib.sha256()
    src = os.path.join(ROOT, "nvfp4_token_quant_amd", "csrc")
    for name in sorted(os.listdir(src)):
        d.update(name.encode())
        with open(os.path.join(src, name), "rb") as f:
            d.update(f.read())
    return d.hexdigest()


def measured_traffic(workload, T, stage):
    """HBM bytes per launch of one stage, from the profiler's FETCH_SIZE and
    WRITE_SIZE counters scaled by a plain copy of known size, as recorded in
    profiles/hbm_traffic.json; None when no record exists for this workload
    or the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_digest():
        return None
    e = rec.get("stages", {}).get(f"{workload}|T={T}|{stage}")
    return None if e is None else e["fetch_bytes"] + e["write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="time this workload alone (default: the decode layer plus every config)")
    ap.add_argument("--T", type=int, default=None, help="tokens (default: the layer's)")
    ap.add_argument("--fast-finalize", action="store_true",
                    help="atomic (non-deterministic) finalize instead of the slot-ordered one")
    ap.add_argument("--rotate", type=int, default=2, help="copies of the expert weights")
    ap.add_argument("--shared", choices=["sum", "average"], default=None,
                    help="add a shared expert (weights of E + 1 experts), combined as routed + shared "
                         "or their average")
    ap.add_argument("--w4a16", action="store_true",
                    help="bf16 activations (no activation quantization), NVFP4 weights")
    ap.add_argument("--prequantized", action="store_true",
                    help="time the forward on activations already quantized per token (codes, block "
                         "scales, global scales made once before timing), the runner contract")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--config-cpu-budget-s", type=float, default=4.0,
                    help="CPU-oracle budget of each entry of the configs list")
    ap.add_argument("--no-configs", action="store_true",
                    help="default run: only the decode headline, without the configs list")
    ap.add_argument("--eager", action="store_true",
                    help="launch the kernels directly instead of replaying captured HIP graphs")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain device copy of 256 MiB, `steps` times (the known-size "
                         "kernel that scales the profiler's HBM byte counters)")
    return ap.parse_args()


class Hip:
    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.h.hipEventSynchronize.argtypes = [P]
        self.h.hipEventDestroy.argtypes = [P]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


CONFIGS = [(1, 16), (3, 4096), (4, None), (5, 1), (5, 7), (5, 2048)]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X; no collectives are built)", file=sys.stderr)
        sys.exit(2)
    if args.prequantized and args.w4a16:
        print("--prequantized applies to NVFP4 activations; --w4a16 takes bf16 ones", file=sys.stderr)
        sys.exit(2)
    import torch

    from nvfp4_token_quant_amd import binding, synth

    if args.copy_reference:
        return copy_reference(args)
    binding.lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(torch.device("cuda:0"))
    if args.layer is not None:
        res = bench_quantize(args, args.T, args.cpu_budget_s) if args.layer == 4 else \
            bench_layer(args, args.layer, args.T or synth.LAYERS[args.layer].T, args.cpu_budget_s)
        print(json.dumps(res), flush=True)
        return
    res = bench_layer(args, 2, synth.LAYERS[2].T, args.cpu_budget_s)
    if not args.no_configs:
        configs = []
        for lid, T in CONFIGS:
            e = bench_quantize(args, T, args.config_cpu_budget_s) if lid == 4 else \
                bench_layer(args, lid, T, args.config_cpu_budget_s)
            configs.append({key: e[key] for key in ("config", "value", "unit", "ms_per_step", "eager_ms_per_step",
                                                   "roofline", "layer_roofline", "cpu_baseline") if key in e})
            print(f"bench: {e['config']['workload']} T={e['config']['T']}: {e['ms_per_step']:.4f} ms/step, "
                  f"{e['roofline']['bound']} frac {e['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
        res["configs"] = configs
    print(json.dumps(res), flush=True)


_WEIGHT_CACHE = {}


def layer_weights(layer_id, n_experts, rotate, dev):
    """Packed weights of a layer, `rotate` copies, kept for the next entry of
    the same layer (the large layer is timed at three batch sizes)."""
    import torch

    from nvfp4_token_quant_amd.workloads import gpu_weights
    key = (layer_id, n_experts, rotate)
    if key not in _WEIGHT_CACHE:
        _WEIGHT_CACHE.clear()
        torch.cuda.empty_cache()
        w = [gpu_weights(layer_id, device=dev, n_experts=n_experts)]
        for _ in range(rotate - 1):
            w.append(w[0].clone())
        _WEIGHT_CACHE[key] = w
    return _WEIGHT_CACHE[key]


def bench_layer(args, layer_id, T, cpu_budget_s):
    """One MoE-layer workload: the timed forwards, their stage rooflines and
    the oracle baseline; returns the result record."""
    import numpy as np
    import torch

    from nvfp4_token_quant_amd import binding, synth
    from nvfp4_token_quant_amd.workloads import to_device_bf16

    L = synth.LAYERS[layer_id]
    H, I, E, k = L.H, L.I, L.E, L.k
    dev = torch.device("cuda:0")
    print(f"bench: layer {layer_id} ({L.name}) T={T} H={H} E={E} k={k} I={I}", file=sys.stderr, flush=True)

    x_bits = synth.activations(layer_id, T)
    logits_np = synth.router_logits(layer_id, T)
    x = to_device_bf16(x_bits, dev)
    logits = torch.from_numpy(logits_np).to(dev)
    n_shared = 1 if args.shared else 0
    weights = layer_weights(layer_id, E + n_shared, args.rotate, dev)
    det = not args.fast_finalize
    max_tokens = max(T, L.max_tokens)
    layers = []
    for w in weights:
        ly = binding.MoeLayer(max_tokens, H, I, E, k, deterministic=det, shared_expert=args.shared,
                              w4a16=args.w4a16)
        ly.bind(w)
        layers.append(ly)
    out = torch.empty_like(x)
    if args.prequantized:
        xq = binding.quantize_per_token(x)   # the handed-over activations (outside the timed region)

    def fwd(ly):
        if args.prequantized:
            ly.forward_quantized_into(*xq, logits, out)
        else:
            ly.forward_into(x, logits, out)
    torch.cuda.synchronize()

    # routing statistics for the algorithmic byte / FLOP counts, from the GPU's own counts
    fwd(layers[0])
    torch.cuda.synchronize()
    counts = layers[0].read_buffer("COUNTS", torch.int32, (E,)).cpu().numpy()
    active = int((counts > 0).sum()) + n_shared  # the shared expert counts as one more active expert
    R = T * (k + n_shared)  # expanded rows through the GEMMs
    w13_bytes = 2 * I * H * 0.5625 + 4
    w2_bytes = H * I * 0.5625 + 4
    stage_bytes = {
        "prologue": (0 if args.prequantized else T * H * 2 + T * (H * 0.5625 + 4)) + T * E * 4 + T * k * 8,
        "gemm1": active * w13_bytes + R * (H * 0.5625 + 4),
        "gemm2": active * w2_bytes,
        "finalize": T * H * 2,
    }
    stage_flops = {"prologue": 0.0, "gemm1": 2.0 * R * 2 * I * H, "gemm2": 2.0 * R * H * I,
                   "finalize": 2.0 * R * H}
    x_bytes = T * (H * 0.5625 + 4) if args.prequantized else T * H * 2
    layer_bytes = active * (w13_bytes + w2_bytes) + x_bytes + T * E * 4 + T * H * 2
    layer_flops = 6.0 * R * I * H

    hip = Hip()
    stages = ["prologue", "gemm1", "gemm2", "finalize"]
    for i in range(args.warmup):
        fwd(layers[i % len(layers)])
    torch.cuda.synchronize()
    lib = binding.lib()
    lib.moe_workspace_set_stage_events.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    def timed_eager():
        """The K forwards launched directly, each recording its five stage
        events on the forward's stream; returns the wall time and the mean
        interval of each stage."""
        evs = [[hip.event() for _ in range(5)] for _ in range(args.steps)]
        arrs = [(ctypes.c_void_p * 5)(*[e.value for e in step]) for step in evs]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ly = layers[i % len(layers)]
            lib.moe_workspace_set_stage_events(ly.handle, arrs[i])
            fwd(ly)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for ly in layers:
            lib.moe_workspace_set_stage_events(ly.handle, None)
        per_stage = {s: [] for s in stages}
        for step in evs:
            for j, s in enumerate(stages):
                per_stage[s].append(hip.elapsed_ms(step[j], step[j + 1]))
        for step in evs:
            for e in step:
                hip.destroy(e)
        return t1 - t0, {s: float(np.mean(v)) for s, v in per_stage.items()}

    eager_ms = None
    if not args.eager:
        # The timed forwards are captured into one HIP graph, the warm-up
        # forwards into another; a decode deployment likewise replays one
        # graph per model step holding every layer.  The graphs hold the
        # kernels only: an event recorded by a HIP graph node keeps the
        # timestamp of its last eager record on every replay (measured), so
        # the stage durations come from the eager timed pass below.
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())

        def capture(n, first):
            with torch.cuda.stream(cap):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for i in range(n):
                        fwd(layers[(first + i) % len(layers)])
            return g

        warm_graph = capture(max(args.warmup, 1), 0)
        graph = capture(args.steps, 0)
        torch.cuda.synchronize()
        warm_graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wall = t1 - t0
        # the same forwards launched directly with their stage events: the
        # second timed region, which gives each kernel's mean duration
        eager_wall, mean_ms = timed_eager()
        eager_ms = eager_wall * 1e3 / args.steps
    else:
        wall, mean_ms = timed_eager()
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T * args.steps / wall

    dominant = max(["gemm1", "gemm2"], key=lambda s: mean_ms[s])
    workload = f"nvfp4_moe_layer_{L.name}" + (f"_shared_{args.shared}" if args.shared else "") + \
        ("_w4a16" if args.w4a16 else "") + ("_prequantized" if args.prequantized else "")
    traffic = measured_traffic(workload, T, dominant)
    mfma_bound = layer_flops / (MFMA_F16_PEAK_TFLOPS * 1e12) > layer_bytes / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = stage_flops[dominant] / (mean_ms[dominant] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": traffic, "kernel": dominant}
    else:
        achieved = stage_bytes[dominant] / (mean_ms[dominant] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dominant}
    layer_time_s = ms_per_step * 1e-3
    layer_roof = {
        "bytes": layer_bytes, "flops": layer_flops,
        "hbm_frac": layer_bytes / layer_time_s / (HBM_PEAK_GBS * 1e9),
        "mfma_frac": layer_flops / layer_time_s / (MFMA_F16_PEAK_TFLOPS * 1e12),
        "stage_ms": mean_ms, "active_experts": active,
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, layer_id, x_bits, T, H, I, k, L.E, cpu_budget_s)

    for ly in layers:
        ly.close()
    result = {
        "metric": "NVFP4 MoE layer tokens/s + % roofline (HBM GB/s decode, MFMA prefill)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "eager_ms_per_step": eager_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 activations, nvfp4 weights, bf16 MFMA, f32 accumulate" if args.w4a16 else
                  "nvfp4 (e2m1 + e4m3 block-16 + f32 global) operands, f16 MFMA, f32 accumulate"),
        "data": "synthetic (seeded; weights from Philox4x64-10, quantized on the device)",
        "config": {"workload": workload, "layer_id": layer_id, "T": T, "H": H,
                   "E": E, "top_k": k, "I": I, "finalize": "deterministic" if det else "atomic",
                   "shared_expert": args.shared,
                   "activations": "bf16 (W4A16)" if args.w4a16 else
                   ("nvfp4, quantized before the forward" if args.prequantized else "nvfp4"),
                   "weights_rotated": args.rotate,
                   "hip_graph": "one graph holding the timed forwards" if not args.eager else "none (eager)",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "cpu_baseline": cpu,
    }
    return result


def copy_reference(args):
    """A plain 256 MiB device-to-device copy (reads and writes 256 MiB each)."""
    import torch

    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": n, "copies": args.steps}), flush=True)


def bench_quantize(args, T, cpu_budget_s):
    """Quantize-only workload: one step = one nvfp4_quantize_per_token launch
    over x bf16 [T, H] (read 2 B, write 0.5625 B per element + 4 B per row);
    returns the result record."""
    import numpy as np
    import torch

    from nvfp4_token_quant_amd import binding, synth
    from nvfp4_token_quant_amd.workloads import to_device_bf16

    L = synth.LAYERS[4]
    T = T or L.T
    H = L.H
    dev = torch.device("cuda:0")
    print(f"bench: layer 4 ({L.name}) T={T} H={H}", file=sys.stderr, flush=True)
    x_bits = synth.activations(4, T)
    nrot = max(1, args.rotate)
    xs = [to_device_bf16(x_bits, dev) for _ in range(nrot)]
    outs = [(torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
             torch.empty((T, H // 16), dtype=torch.uint8, device=dev),
             torch.empty((T,), dtype=torch.float32, device=dev)) for _ in range(nrot)]
    for i in range(args.warmup):
        binding.quantize_per_token_into(xs[i % nrot], *outs[i % nrot])
    torch.cuda.synchronize()
    # one event pair on the launching stream around the timed launches (back
    # to back, nothing else on the stream): their mean duration
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        binding.quantize_per_token_into(xs[i % nrot], *outs[i % nrot])
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = T * H * 2 + T * H // 2 + T * H // 16 + 4 * T
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_quantize(x_bits, cpu_budget_s)
    result = {
        "metric": "NVFP4 MoE layer tokens/s + % roofline (HBM GB/s decode, MFMA prefill)",
        "value": T * args.steps / (t1 - t0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 in; e2m1 + e4m3 + f32 out)",
        "data": "synthetic (seeded Student-t(3) rows, every 97th row zero, 4 rows x1e3)",
        "config": {"workload": "nvfp4_quantize_per_token", "layer_id": 4, "T": T, "H": H,
                   "inputs_rotated": nrot, "hip_graph": False, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("nvfp4_quantize_per_token", T, "quantize_rows"),
                     "kernel": "quantize_rows",
                     "kernel_ms": kernel_ms, "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
    }
    return result


def cpu_baseline_quantize(x_bits, budget_s):
    """The oracle's per-row quantizer, as it stands, on a bounded sample of rows."""
    import oracle

    T = x_bits.shape[0]
    n = min(T, 256)
    oracle.quantize_rows(x_bits[:n])
    t0 = time.perf_counter()
    oracle.quantize_rows(x_bits[:n])
    per_row = (time.perf_counter() - t0) / n
    n = int(min(T, max(n, budget_s / max(per_row, 1e-9))))
    reps, dt = 0, 0.0
    while dt < budget_s * 0.8 or reps == 0:
        t0 = time.perf_counter()
        oracle.quantize_rows(x_bits[:n])
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {n} of {T} rows x {reps} repetitions ({dt:.1f} s)"}


def cpu_baseline(args, layer_id, x_bits, T, H, I, k, E, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload:
    tokens of the batch (all of it if the budget allows), the whole forward
    in binary64 with the expert weights prepared before timing, repeated to
    about budget_s.  On the large layer the sample is at most 8 tokens (each
    of its experts costs the oracle about a second to prepare)."""
    import numpy as np

    import oracle
    from nvfp4_token_quant_amd import synth
    from tests.layer_fixtures import oracle_expert, oracle_weights

    ids, w = oracle.router(synth.router_logits(layer_id, T), k)
    shared = None
    if args.shared:
        shared = oracle.QuantWeights(np.array([E], np.int32), *(a[None] for a in oracle_expert(layer_id, E)))

    xq = oracle.quantize_rows(x_bits) if args.prequantized else None

    def run(toks, qw):
        if xq is not None:
            return oracle.moe_layer_quantized(*xq, ids, w, toks, H, I, qw)
        if shared is None:
            return oracle.moe_layer(x_bits, ids, w, toks, H, I, qw, a16=args.w4a16)
        return oracle.moe_layer_shared(x_bits, ids, w, toks, H, I, qw, shared, args.shared, a16=args.w4a16)
    rng = np.random.default_rng(0)
    cap = 8 if H * I >= 7168 * 2048 else T
    toks = np.arange(T)
    # grow the sample until it costs about budget_s (the oracle is linear in tokens)
    probe = toks[: max(1, min(T, 4))]
    qw = oracle_weights(layer_id, np.unique(ids[probe]))
    t0 = time.perf_counter()
    run(probe, qw)
    t_probe = time.perf_counter() - t0
    n = int(min(T, cap, max(len(probe), budget_s / max(t_probe / len(probe), 1e-6))))
    toks = np.sort(rng.choice(T, n, replace=False)) if n < T else toks
    qw = oracle_weights(layer_id, np.unique(ids[toks]))
    reps, dt = 0, 0.0
    while dt < budget_s * 0.8 or reps == 0:   # repeat small samples to ~the budget
        t0 = time.perf_counter()
        run(toks, qw)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * len(toks) / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(toks)} of {T} tokens of the same layer x {reps} repetitions, full "
                      f"forward in binary64 ({dt:.1f} s; weights prepared before timing)"}


if __name__ == "__main__":
    main()
