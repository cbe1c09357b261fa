"""Benchmark of the MoE layer forward on one MI355X.

Default workload: the OLMoE-1B-7B-shaped layer (d=2048, E=64, k=8, SwiGLU
ffn=1024, bf16, softmax top-k without renorm, router skew bias std 0.5) at
T=4096 tokens, seeded synthetic inputs resident in HBM.  A step is one
moe_forward: router + top-k, permutation, gate/up GEMM, down GEMM, combine.

Prints one JSON line.  `roofline` is for the dominant kernel (the grouped
gate/up SwiGLU GEMM, MFMA-bound), timed with HIP events recorded by the
library around that launch on its own stream during the timed steps.
`cpu_baseline` is the FP64 oracle on a bounded token sample of the same
workload.  `decode` adds the same layer at decode sizes (hipGraph replays,
weights rotated over several copies so the Infinity Cache does not serve
them), reported against HBM bandwidth.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=4096)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                    help="expert weight layout (tiled: repacked once before timing)")
    ap.add_argument("--decode-only", action="store_true", help="run only the decode sweep and print it")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/gateup_tiled_olmoe_T4096_traffic.json from four rocprofv3 --pmc csv "
                         "directories (FETCH_SIZE and WRITE_SIZE of this bench, then of --copy-probe) and exit")
    ap.add_argument("--profile-layer", metavar="SPEC",
                    help="run --warmup + --steps eager forwards of the named synthetic layer at --T tokens "
                         "(for counter passes on one layer's kernels), print the mean ms and exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device-to-device copy three times (calibrates the HBM byte counters)")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    # reference points for HBM: read+write bandwidth of a plain copy, read bandwidth of a reduction
    big = torch.ones(4 << 28, dtype=torch.float32, device="cuda")  # 4 GiB
    big.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        big.sum()
    e1.record()
    torch.cuda.synchronize()
    ms_r = e0.elapsed_time(e1) / 3
    print(json.dumps({"copy_probe_bytes": a.numel() * 4, "copies": 3, "ms_per_copy": round(ms, 3),
                      "read_plus_write_GBps": round(2 * a.numel() * 4 / (ms * 1e-3) / 1e9, 1),
                      "reduction_read_GBps": round(big.numel() * 4 / (ms_r * 1e-3) / 1e9, 1)}))


class HipEvents:
    """hipEvent_t handles created through the HIP runtime (for the library's timing hook)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b])) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return f.value

    def slice(self, i, n):
        return ctypes.cast(ctypes.byref(self.ev, i * ctypes.sizeof(ctypes.c_void_p)), ctypes.POINTER(ctypes.c_void_p))

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


def moe_layer(sp, lay, layout):
    """A MoeLayer over the generated weights; with layout "tiled" the expert
    matrices are repacked once (moe_pack_weights), before any timing."""
    from mixture_experts_layer_13_amd import binding as B
    from mixture_experts_layer_13_amd.layer import MoeLayer
    cfg = B.make_cfg(1, sp.d, sp.E, sp.k, sp.ffn, sp.n_shared, sp.ffn_shared, act=sp.act, expert=sp.expert,
                     score=sp.score, renorm=sp.renorm, gate_scale=sp.gate_scale, capacity=sp.capacity,
                     layout=layout, groups=sp.groups)
    mats = [lay.w_gate, lay.w_up, lay.w_down, lay.sh_gate, lay.sh_up, lay.sh_down]
    if layout == "tiled":
        mats = [None if m is None else B.pack_tiled(m, sp.expert) for m in mats]
    wg, wu, wd, shg, shu, shd = mats
    return MoeLayer(cfg, lay.w_router, wg, wu, wd, logit_bias=lay.logit_bias, select_bias=lay.select_bias,
                    s_gate=lay.s_gate, s_up=lay.s_up, s_down=lay.s_down, sh_gate=shg, sh_up=shu, sh_down=shd)


def expert_bytes(sp):
    n = 3 * sp.d * sp.ffn
    if sp.expert == "int4":
        return n // 2 + (3 * sp.d * sp.ffn // 128) * 2
    if sp.expert == "fp8":  # one byte per weight and an fp32 scale per output channel
        return n + (2 * sp.ffn + sp.d) * 4
    return n * (4 if sp.expert == "f32" else 2)


def alg_work(sp, T, idx, drop):
    """Algorithmic bytes and flops of one forward: touched expert weights, shared
    experts, router weight, x and out; flops 6 d F per kept pair + 6 d Fs S T + 2 T d E."""
    import torch
    kept = (drop == 0)
    touched = int(torch.unique(idx[kept]).numel()) if kept.any() else 0
    n_kept = int(kept.sum().item())
    es = 4 if sp.act == "f32" else 2
    byts = (touched * expert_bytes(sp) + sp.n_shared * 3 * sp.d * sp.ffn_shared * es + sp.E * sp.d * es
            + 2 * T * sp.d * es)
    gateup = 4.0 * sp.d * sp.ffn * n_kept + 4.0 * sp.d * sp.ffn_shared * sp.n_shared * T
    flops = 1.5 * gateup + 2.0 * T * sp.d * sp.E
    return dict(bytes=byts, flops=flops, gateup_flops=gateup, touched=touched, kept=n_kept)


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "gateup_tiled_olmoe_T4096_traffic.json")
# the sources the dominant (bf16 tiled gate/up) kernel is compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_13_amd", "csrc", f)
                  for f in ("ffn_tiled.hip", "ffn_common.hpp", "common.hpp", "kernels.hpp")]


def kernel_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_record():
    """HBM bytes of the dominant kernel from the committed rocprofv3 counter summary,
    valid only while the kernel's sources are the ones the counters were taken on."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    rec = json.load(open(TRAFFIC_PATH))
    if rec.get("source_sha256") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_mean_kib(csv_dir, counter, kernel_substr, largest=None):
    """Mean per-dispatch value of `counter` over the dispatches of kernels whose
    name contains one of `kernel_substr` in a rocprofv3 --pmc csv output directory
    (over the `largest` biggest values only, when given)."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and any(k in r["Kernel_Name"] for k in kernel_substr):
                vals.append(float(r["Counter_Value"]))
    if largest:
        vals = sorted(vals)[-largest:]
    if not vals:
        raise SystemExit(f"no {counter} values for kernels matching {kernel_substr!r} under {csv_dir}")
    return sum(vals) / len(vals)


def write_traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    """Writes the traffic record of the gate/up kernel from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the bench, and of the copy probe,
    whose known 1 GiB read + 1 GiB write calibrates each counter."""
    gu = ("ffn_tiled32_kernel<true", "ffn_tiled32_kernelILb1E")  # demangled or mangled name
    copy = ("copyBuffer",)  # the runtime's device-to-device copy kernel behind the probe's Tensor.copy_
    f_k = _pmc_mean_kib(fetch_dir, "FETCH_SIZE", gu)
    w_k = _pmc_mean_kib(write_dir, "WRITE_SIZE", gu)
    cf = _pmc_mean_kib(copy_fetch_dir, "FETCH_SIZE", copy, largest=3)
    cw = _pmc_mean_kib(copy_write_dir, "WRITE_SIZE", copy, largest=3)
    nbytes = 1 << 30
    fs, ws = nbytes / (cf * 1024), nbytes / (cw * 1024)
    rec = {"kernel": "ffn_tiled32_kernel<gate/up + SwiGLU, tiled weights>", "workload": "olmoe_1b7b_layer_T4096",
           "fetch_size_kib_per_launch": round(f_k, 1), "write_size_kib_per_launch": round(w_k, 1),
           "copy_probe": {"bytes_read": nbytes, "bytes_written": nbytes, "fetch_size_kib": round(cf, 1),
                          "write_size_kib": round(cw, 1), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
           "hbm_bytes_per_launch": int(f_k * 1024 * fs + w_k * 1024 * ws),
           "commands": commands, "source_files": [os.path.relpath(f, ROOT) for f in KERNEL_SOURCES],
           "source_sha256": kernel_sha()}
    with open(TRAFFIC_PATH, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def cpu_baseline(sp, lay, x, n_tokens, min_s=10.0):
    import oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_harness import ExpertSource, to_f64
    xs = x[:n_tokens]
    xf, wr, lb = to_f64(xs), to_f64(lay.w_router), to_f64(lay.logit_bias)

    class HostWeights:  # expert weights copied to host memory before timing (inputs resident)
        w_gate = [t.cpu() for t in lay.w_gate]
        w_up = [t.cpu() for t in lay.w_up]
        w_down = [t.cpu() for t in lay.w_down]

    host = ExpertSource(sp, HostWeights)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    # whole runs of the sample until at least `min_s` seconds of host time (at most 20 runs)
    runs, t0 = 0, time.perf_counter()
    while runs < 20 and (runs == 0 or time.perf_counter() - t0 < min_s):
        O.moe_layer(xf, wr, host, sp.E, sp.k, score=sp.score, renorm=sp.renorm, gate_scale=sp.gate_scale,
                    logit_bias=lb, capacity=sp.capacity)
        runs += 1
    dt = time.perf_counter() - t0
    return {"value": runs * n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_tokens} of the {x.shape[0]} tokens (full FP64 layer on the sample: routing, "
                      f"all selected expert FFNs from bf16 bit patterns, combine), {runs} runs in {dt:.1f} s"}


def clone_weights(lay):
    """A copy of a layer with every weight tensor in new device memory."""
    import dataclasses
    kw = {f.name: getattr(lay, f.name).clone() for f in dataclasses.fields(lay)
          if f.name != "spec" and getattr(lay, f.name) is not None}
    return dataclasses.replace(lay, **kw)


def decode_sweep(sp, lay, layout, Ts=(1, 8, 32, 64), replays=200, copies=4, name="olmoe_1b7b"):
    """Decode-sized forwards as hipGraph replays over `copies` weight copies (cold in
    the 256 MB Infinity Cache), reported as achieved HBM bandwidth."""
    import torch

    import moe_synth as S
    layers = [moe_layer(sp, lay, layout)]
    for c in range(1, copies):
        layers.append(moe_layer(sp, clone_weights(lay), layout))
    res = {}
    s = torch.cuda.Stream()
    for T in Ts:
        x = S.make_tokens(sp, T, device="cuda")
        # the weights, their packing and x were made on the default stream: finish them before
        # anything runs on `s`
        torch.cuda.synchronize()
        graphs, outs = [], []
        for ml in layers:
            o = (torch.empty((T, sp.d), dtype=ml.act_dtype, device="cuda"),
                 torch.empty((T, sp.k), dtype=torch.int32, device="cuda"),
                 torch.empty((T, sp.k), dtype=torch.float32, device="cuda"),
                 torch.empty((T, sp.k), dtype=torch.uint8, device="cuda"))
            ml.workspace(ml.cfg_for(T))
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                ml.forward(x, *o)  # eager warm-up on the capture stream
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                ml.forward(x, *o)
            graphs.append(g)
            outs.append(o)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(replays):
            graphs[i % len(graphs)].replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / replays
        w = alg_work(sp, T, outs[0][1], outs[0][3])
        gbs = w["bytes"] / (us * 1e-6) / 1e9
        res[f"T{T}"] = {"us_per_layer": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
                        "alg_bytes": w["bytes"], "touched_experts": w["touched"], "hbm_GBps": round(gbs, 1),
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del graphs
    return {"layer": name, "method": f"hipGraph replay, {copies} weight copies round-robin, {replays} replays",
            "points": res}


def decode_other(layout):
    """The other decode-sized layers the HBM target covers: Qwen3 INT4 at T=32 (4
    copies of its 0.31 GB of expert weights) and DeepSeek-V3 at T=1 and 16 (2 copies:
    one token already touches 0.8 GB), plus DeepSeek-V3 T=256 from its token sweep,
    and the OLMoE-shaped layer with FP8 experts (half the bf16 bytes) at T=1..64."""
    import torch

    import moe_synth as S
    out = {}
    for name, Ts, copies in (("qwen3_int4", (32,), 4), ("dsv3", (1, 16, 256), 2), ("olmoe_fp8", (1, 8, 32, 64), 4)):
        sp = S.SPECS[name]
        lay = S.make_layer(sp, device="cuda")
        out[name] = decode_sweep(sp, lay, layout, Ts=Ts, replays=100, copies=copies, name=name)
        del lay
        torch.cuda.empty_cache()
    return out


LAUNCHES = ["router", "permute", "gateup", "down", "combine"]


def time_layer(ml, x, steps, warmup):
    """Eager forwards: `warmup` untimed, then `steps` timed between two events on
    the stream, with the library's per-launch HIP events recorded on the same
    stream.  Returns ms per step, mean ms per launch, the last outputs, launches."""
    import torch

    from mixture_experts_layer_13_amd import binding as B
    T = x.shape[0]
    c = ml.cfg
    nl = B.forward_launches(ml.cfg_for(T))
    outs = (torch.empty((T, c.d), dtype=ml.act_dtype, device="cuda"),
            torch.empty((T, c.k), dtype=torch.int32, device="cuda"),
            torch.empty((T, c.k), dtype=torch.float32, device="cuda"),
            torch.empty((T, c.k), dtype=torch.uint8, device="cuda"))
    for _ in range(warmup):
        ml.forward(x, *outs)
    torch.cuda.synchronize()
    ev = HipEvents(steps * (nl + 1))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        B.lib.moe_set_timing_events(ev.slice(i * (nl + 1), nl + 1), nl + 1)
        ml.forward(x, *outs)
    t1.record()
    B.lib.moe_set_timing_events(None, 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps
    per = {n: 0.0 for n in LAUNCHES[:nl]}
    for i in range(steps):
        b = i * (nl + 1)
        for j, n in enumerate(LAUNCHES[:nl]):
            per[n] += ev.ms(b + j, b + j + 1) / steps
    ev.close()
    return ms_step, per, outs, nl, wall


def prefill_sweep(layout, steps=20, warmup=3):
    """The prefill layers the MFMA target is set for (T >= 8192), and the INT4
    layer's prefill: useful-flop MFMA fraction of the whole layer and of its
    gate/up launch."""
    import torch

    import moe_synth as S
    res = {}
    # DeepSeek-V3 also at T=4096, the step of its token sweep below the prefill target
    for name, Ts in (("dsv2_lite", (8192,)), ("dsv2_lite_cap", (8192,)), ("dsv3", (4096, 16384)),
                     ("qwen3_int4", (4096,))):
        sp = S.SPECS[name]
        lay = S.make_layer(sp, device="cuda")
        ml = moe_layer(sp, lay, layout)
        for T in Ts:
            x = S.make_tokens(sp, T, device="cuda")
            ms, per, outs, _, _ = time_layer(ml, x, steps, warmup)
            w = alg_work(sp, T, outs[1], outs[3])
            res[f"{name}_T{T}"] = {
                "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                "mfma_frac_layer": round(w["flops"] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "mfma_frac_gateup": round(w["gateup_flops"] / (per["gateup"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "per_launch_us": {n: round(v * 1e3, 2) for n, v in per.items()},
                "kept_pairs": w["kept"], "pairs": T * sp.k}
            del x, outs
        del ml, lay
        torch.cuda.empty_cache()
    return {"method": f"eager, {steps} timed forwards after {warmup}; useful flops only (dropped pairs and tile "
                      "padding excluded)", "points": res}


def main():
    args = parse()
    if args.traffic_record:
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d <out> -o pmc -- python3 bench.py {a}"
                for a in ("--steps 5 --warmup 2 --no-cpu --no-decode --no-prefill", "--copy-probe")
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        write_traffic_record(*args.traffic_record, commands=cmds)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the layer on one GPU only (asked for {max(args.gpus, world)}): the path has no "
              "multi-GPU mode (expert-parallel sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_synth as S
    from mixture_experts_layer_13_amd import binding as B

    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.profile_layer:
        psp = S.SPECS[args.profile_layer]
        play = S.make_layer(psp, device="cuda")
        ml = moe_layer(psp, play, args.layout)
        x = S.make_tokens(psp, args.T, device="cuda")
        ms = time_layer(ml, x, args.steps, args.warmup)[0]
        print(json.dumps({"layer": args.profile_layer, "T": args.T, "ms_per_forward": round(ms, 4)}), flush=True)
        return
    sp = S.SPECS["olmoe"]
    T = args.T
    lay = S.make_layer(sp, device="cuda")
    if args.decode_only:
        print(json.dumps(decode_sweep(sp, lay, args.layout)), flush=True)
        print(json.dumps(decode_other(args.layout)), flush=True)
        return
    x = S.make_tokens(sp, T, device="cuda")
    ml = moe_layer(sp, lay, args.layout)
    K = args.steps
    ms_step, per, outs, nl, wall = time_layer(ml, x, K, args.warmup)

    w = alg_work(sp, T, outs[1], outs[3])
    t_gu = per["gateup"] * 1e-3
    achieved = w["gateup_flops"] / t_gu / 1e12
    traffic = traffic_record()
    line = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"olmoe_1b7b_layer_T{T}", "T": T, "d": sp.d, "E": sp.E, "k": sp.k,
                   "ffn": sp.ffn, "launches_per_layer": nl, "weight_layout": args.layout},
        "roofline": {"bound": "mfma", "kernel": "ffn_tiled32_kernel<gate/up + SwiGLU>", "achieved": round(achieved, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "avg_launch_us": round(per["gateup"] * 1e3, 2),
                     "alg_flops_per_launch": w["gateup_flops"]},
        "layer": {"per_launch_us": {n: round(v * 1e3, 2) for n, v in per.items()},
                  "alg_flops": w["flops"], "alg_bytes": w["bytes"],
                  "mfma_frac": round(w["flops"] / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "wall_s_timed": round(wall, 3)},
    }
    if not args.no_decode:
        line["decode"] = decode_sweep(sp, lay, args.layout)
        line["decode_other"] = decode_other(args.layout)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(sp, lay, x, n_tokens=T)  # the whole workload, ~10 s of host time
    if not args.no_prefill:
        del ml, lay, x
        torch.cuda.empty_cache()
        line["prefill"] = prefill_sweep(args.layout)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
