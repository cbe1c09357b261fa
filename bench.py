"""Benchmark of the MoE layer forward on one MI355X.

Headline workload: the DeepSeek-V3-shaped layer (d=7168, 256 routed experts,
k=8, one shared expert, SwiGLU ffn=2048, bf16, sigmoid scoring with a
selection-only bias, gates 2.5 x renormalised) at T=16384 tokens, the largest
configuration and the one the prefill MFMA target is set on.  Seeded synthetic
inputs and random-init weights of that shape are resident in HBM.  A step is
one moe_forward: router + top-k, permutation, gate/up GEMM, down GEMM, combine.

Prints one JSON line.  `roofline` is for the dominant kernel (the grouped
gate/up SwiGLU GEMM, MFMA-bound), timed with HIP events recorded by the
library around that launch on its own stream during the timed steps.
`cpu_baseline` is the FP64 oracle: routing over every token plus the whole
layer on a seeded 1024-token subset, extrapolated to the workload.  Sub-keys:
the OLMoE-shaped layer at T=4096 (`olmoe_T4096`), decode sizes as hipGraph
replays with weights rotated over several copies so the Infinity Cache does
not serve them, several layer forwards per graph as a model's captured decode
step holds its layers, and one per graph beside it (`decode`, `decode_other`,
against HBM bandwidth), the other
prefill layers (`prefill`), routing near-ties and INT4 drift (`routing`), and the
memory-system probe rates the kernels are read against (`memory_probe`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-prefill]
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
FP8_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA (layers with FP8 weights and FP8 activations)
METRIC = "MoE-layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak"


# The pages' own figures, quoted with the hardware they state, as context for the numbers above;
# none of them is a target or a baseline of this bench (other hardware, other software).
PAGES_CONTEXT = {
    "launch_bound_study": {
        "source": "picx.dev summary of the MoE launch-bound study: Summary (key finding 1) and "
                  "Empirical Validation / Triton Kernel Results",
        "fused_kernels_isolated_speedup": "5.6x-9.0x", "end_to_end_speedup": "0.999x",
        "amdahl_ceiling": "1.072x (7.87% of the forward in the fused modules)",
        "olmoe_latency_128_to_4096_tokens_ms": [246.8, 383.4],
        "hardware": "NVIDIA A100 (the isolated kernel benchmark); eager PyTorch forwards of ~1000 launches",
    },
    "ridge": {
        "source": "MoE at the inference level: routing overhead, load balancing, expert parallelism, and "
                  "the memory-bandwidth story -- Arithmetic intensity",
        "flop_per_byte": 295, "hardware": "NVIDIA H100 SXM",
        "this_gpu_flop_per_byte": {"bf16": BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3,
                                   "fp8": FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3},
    },
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=16384, help="tokens of the headline (or --profile-layer) workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                    help="expert weight layout (tiled: repacked once before timing)")
    ap.add_argument("--decode-only", action="store_true", help="run only the decode sweep and print it")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the gate/up traffic record of --traffic-workload under profiles/ from four "
                         "rocprofv3 --pmc csv directories (FETCH_SIZE and WRITE_SIZE of --profile-layer runs, then "
                         "of --copy-probe) and exit")
    ap.add_argument("--traffic-workload", choices=sorted(TRAFFIC_WORKLOADS), default="dsv3_T16384")
    ap.add_argument("--profile-layer", metavar="SPEC",
                    help="run --warmup + --steps eager forwards of the named synthetic layer at --T tokens "
                         "(for counter passes on one layer's kernels), print the mean ms and exit")
    ap.add_argument("--memory-probe", action="store_true",
                    help="print the streaming-read and global->LDS probe rates and exit")
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


def memory_probe():
    """Ceilings the kernels are read against, from the probe library (csrc/probe.hip):
    a streaming read of 4 GiB (ordinary and non-temporal 16-byte loads; the best over
    grid sizes), and direct global -> LDS loads from an L2-resident 4 MiB span and from
    a 4 GiB span, as a stream of whole KB per wave-wide load or as 64-byte pieces of 16
    rows walking along the rows (each 128-byte line read in two halves, so the second
    half of every line comes from cache even over the 4 GiB span)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mixture_experts_layer_13_amd", "libmoe_probe.so"))
    P = ctypes.c_void_p
    lib.moe_probe_stream_read.argtypes = [P, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, P, P]
    lib.moe_probe_dma_read.argtypes = [P, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    nbytes = 4 << 30
    buf = torch.full((nbytes // 4,), 1, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = P(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=3):
        assert fn() == 0
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            assert fn() == 0
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    res = {}
    for nt, name in ((0, "stream_read_GBps"), (1, "stream_read_nontemporal_GBps")):
        best = 0.0
        for blocks in (1024, 2048, 4096, 8192):
            t = timed(lambda: lib.moe_probe_stream_read(P(buf.data_ptr()), nbytes, nt, blocks, P(sink.data_ptr()),
                                                        stream))
            best = max(best, nbytes / t / 1e9)
        res[name] = round(best, 1)
    steps, blocks = 256, 8192
    moved = blocks * 4 * steps * 8192
    for span, tag in ((4 << 20, "l2"), (nbytes, "hbm")):
        for gather in (0, 1):
            t = timed(lambda: lib.moe_probe_dma_read(P(buf.data_ptr()), span, gather, steps, blocks, stream))
            res[f"dma_{tag}_{'gather64' if gather else 'contig'}_GBps"] = round(moved / t / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    res["method"] = ("stream: 4 GiB once per launch, 16 loads of 16 B in flight per lane, best of 1024-8192 "
                     "blocks; dma: 8192 blocks x 4 waves x 256 steps x 8 KB, two steps in flight per wave, "
                     "wrapping over the first 4 MiB (l2) or 4 GiB (hbm) of the buffer; contig = consecutive KBs, "
                     "gather64 = 16 rows x 64 B per load, the next 64 B of the same rows at the next step")
    return res


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
                    s_gate=lay.s_gate, s_up=lay.s_up, s_down=lay.s_down, sh_gate=shg, sh_up=shu, sh_down=shd,
                    shs_gate=lay.shs_gate, shs_up=lay.shs_up, shs_down=lay.shs_down)


def expert_bytes(sp, ffn=None):
    ffn = sp.ffn if ffn is None else ffn
    n = 3 * sp.d * ffn
    if sp.expert == "int4":
        return n // 2 + (3 * sp.d * ffn // 128) * 2
    if sp.expert in ("fp8", "fp8a8"):  # one byte per weight and an fp32 scale per output channel
        return n + (2 * ffn + sp.d) * 4
    return n * (4 if sp.expert == "f32" else 2)


def shared_bytes(sp):
    """Bytes of the shared experts (INT4 layers keep bf16 shared experts, FP8 layers FP8 ones)."""
    if not sp.n_shared:
        return 0
    if sp.expert == "int4":
        return sp.n_shared * 3 * sp.d * sp.ffn_shared * 2
    return sp.n_shared * expert_bytes(sp, sp.ffn_shared)


def alg_work(sp, T, idx, drop):
    """Algorithmic bytes and flops of one forward: touched expert weights, shared
    experts, router weight, x and out; flops 6 d F per kept pair + 6 d Fs S T + 2 T d E."""
    import torch
    kept = (drop == 0)
    touched = int(torch.unique(idx[kept]).numel()) if kept.any() else 0
    n_kept = int(kept.sum().item())
    es = 4 if sp.act == "f32" else 2
    byts = touched * expert_bytes(sp) + shared_bytes(sp) + sp.E * sp.d * es + 2 * T * sp.d * es
    gateup = 4.0 * sp.d * sp.ffn * n_kept + 4.0 * sp.d * sp.ffn_shared * sp.n_shared * T
    flops = 1.5 * gateup + 2.0 * T * sp.d * sp.E
    return dict(bytes=byts, flops=flops, gateup_flops=gateup, touched=touched, kept=n_kept)


# gate/up traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE of the bf16 tiled gate/up kernel),
# one per workload: (spec, T, the kernel the plan runs there)
TRAFFIC_WORKLOADS = {"dsv3_T16384": ("dsv3", 16384, "tiled256"), "olmoe_T4096": ("olmoe", 4096, "tiled32")}
# per kernel: its name in the counter csv (demangled or mangled), as reported, and the sources it is compiled from
GATEUP_KERNELS = {
    "tiled32": (("ffn_tiled32_kernel<true", "ffn_tiled32_kernelILb1E"),
                "ffn_tiled32_kernel<gate/up + SwiGLU, tiled weights>", "ffn_tiled.hip"),
    "tiled256": (("ffn_tiled256_kernel<true", "ffn_tiled256_kernelILb1E"),
                 "ffn_tiled256_kernel<gate/up + SwiGLU, tiled weights>", "ffn_tiled256.hip"),
}


def kernel_sources(workload):
    src = GATEUP_KERNELS[TRAFFIC_WORKLOADS[workload][2]][2]
    return [os.path.join(ROOT, "mixture_experts_layer_13_amd", "csrc", f)
            for f in (src, "ffn_common.hpp", "common.hpp", "kernels.hpp")]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"gateup_tiled_{workload}_traffic.json")


def kernel_sha(workload):
    h = hashlib.sha256()
    for f in kernel_sources(workload):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_record(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, valid only while the kernel's sources are the ones the counters were taken on."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_sha(workload):
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


def write_traffic_record(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    """Writes the traffic record of the gate/up kernel from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the workload, and of the copy probe,
    whose known 1 GiB read + 1 GiB write calibrates each counter."""
    copy = ("copyBuffer",)  # the runtime's device-to-device copy kernel behind the probe's Tensor.copy_
    names, label, _ = GATEUP_KERNELS[TRAFFIC_WORKLOADS[workload][2]]
    f_k = _pmc_mean_kib(fetch_dir, "FETCH_SIZE", names)
    w_k = _pmc_mean_kib(write_dir, "WRITE_SIZE", names)
    cf = _pmc_mean_kib(copy_fetch_dir, "FETCH_SIZE", copy, largest=3)
    cw = _pmc_mean_kib(copy_write_dir, "WRITE_SIZE", copy, largest=3)
    nbytes = 1 << 30
    fs, ws = nbytes / (cf * 1024), nbytes / (cw * 1024)
    rec = {"kernel": label, "workload": workload,
           "fetch_size_kib_per_launch": round(f_k, 1), "write_size_kib_per_launch": round(w_k, 1),
           "copy_probe": {"bytes_read": nbytes, "bytes_written": nbytes, "fetch_size_kib": round(cf, 1),
                          "write_size_kib": round(cw, 1), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
           "hbm_bytes_per_launch": int(f_k * 1024 * fs + w_k * 1024 * ws),
           "commands": commands, "source_files": [os.path.relpath(f, ROOT) for f in kernel_sources(workload)],
           "source_sha256": kernel_sha(workload)}
    with open(traffic_path(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def gateup_alg_bytes(sp, T, w):
    """Algorithmic HBM bytes of one gate/up launch: the touched experts' gate and up
    weights, the shared experts' gate and up weights, each token row of x once, h written."""
    es = 2
    wbytes = (w["touched"] * 2 * sp.d * sp.ffn + sp.n_shared * 2 * sp.d * sp.ffn_shared) * es
    return int(wbytes + T * sp.d * es + (w["kept"] * sp.ffn + T * sp.n_shared * sp.ffn_shared) * es)


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(sp, lay, x, n_ffn=None, seed=0, min_s=10.0):
    """The FP64 oracle on the host cores, timed on a bounded sample of the workload.

    n_ffn None: the whole layer over every token, repeated to at least `min_s` s.
    n_ffn = n: routing (router product, scores, top-k, gates, assignment) over every
    token once, and the whole layer once on a seeded subset of n tokens (dropless
    routing is per token, so the subset's routes are those of the full run); the
    workload's time is extrapolated as t_route + t_subset * T / n."""
    import numpy as np

    import oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_harness import ExpertSource, to_f64
    T = x.shape[0]
    xf, wr, lb, sb = to_f64(x), to_f64(lay.w_router), to_f64(lay.logit_bias), to_f64(lay.select_bias)

    class HostWeights:  # every weight copied to host memory before timing (inputs resident)
        pass
    for f in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down"):
        t = getattr(lay, f)
        setattr(HostWeights, f, None if t is None else [m.cpu() for m in t])
    kw = dict(score=sp.score, renorm=sp.renorm, gate_scale=sp.gate_scale, logit_bias=lb, select_bias=sb,
              capacity=sp.capacity, shared=ExpertSource(sp, HostWeights, shared=True) if sp.n_shared else None,
              n_shared=sp.n_shared, groups=sp.groups)
    host = ExpertSource(sp, HostWeights)
    base = {"unit": "tokens/s", "cores": _threads(), "blas_threads": _threads(), "host_cpus": os.cpu_count(),
            "kind": "oracle"}
    if n_ffn is None:
        runs, t0 = 0, time.perf_counter()
        while runs < 20 and (runs == 0 or time.perf_counter() - t0 < min_s):
            O.moe_layer(xf, wr, host, sp.E, sp.k, **kw)
            runs += 1
        dt = time.perf_counter() - t0
        return dict(base, value=runs * T / dt,
                    sample=f"all {T} tokens (full FP64 layer: routing, every selected expert FFN from the stored "
                           f"bit patterns, combine), {runs} runs in {dt:.1f} s")
    assert sp.capacity is None, "the subset extrapolation needs per-token (dropless) routing"
    t0 = time.perf_counter()
    O.moe_layer(xf, wr, host, sp.E, sp.k, ffn_rows=np.arange(0), **kw)
    t_route = time.perf_counter() - t0
    sub = np.sort(np.random.default_rng(seed).choice(T, size=n_ffn, replace=False))
    t0 = time.perf_counter()
    O.moe_layer(xf[sub], wr, host, sp.E, sp.k, **kw)
    t_sub = time.perf_counter() - t0
    est = t_route + t_sub * T / n_ffn
    return dict(base, value=T / est,
                sample=f"routing over all {T} tokens ({t_route:.1f} s) + the whole FP64 layer (routing, every "
                       f"selected expert FFN from the stored bf16 bit patterns, shared expert, combine) on a seeded "
                       f"{n_ffn}-token subset ({t_sub:.1f} s, seed {seed}); value = T / (t_route + t_subset * T / "
                       f"{n_ffn}), i.e. {est:.1f} s for the workload")


def routing_report(ml, sp, x):
    """Near-ties of the route on the GPU's own fp32 selection keys (tokens whose k-th
    and (k+1)-th keys differ by at most 1e-3 / 1e-5), from moe_route's scores."""
    import torch
    _, _, scores = ml.route(x)
    key = scores if ml.select_bias is None else scores + ml.select_bias[None, :]
    if sp.k >= sp.E:
        return {"tokens": x.shape[0], "near_ties_1e-3": 0, "near_ties_1e-5": 0}
    top = torch.topk(key, sp.k + 1, dim=1).values
    margin = top[:, sp.k - 1] - top[:, sp.k]
    return {"tokens": x.shape[0], "near_ties_1e-3": int((margin <= 1e-3).sum()),
            "near_ties_1e-5": int((margin <= 1e-5).sum())}


def clone_weights(lay):
    """A copy of a layer with every weight tensor in new device memory."""
    import dataclasses
    kw = {f.name: getattr(lay, f.name).clone() for f in dataclasses.fields(lay)
          if f.name != "spec" and getattr(lay, f.name) is not None}
    return dataclasses.replace(lay, **kw)


def decode_sweep(sp, lay, layout, Ts=(1, 8, 32, 64), replays=200, copies=4, name="olmoe_1b7b"):
    """Decode-sized forwards as hipGraph replays over `copies` weight copies (cold in
    the 256 MB Infinity Cache), reported as achieved HBM bandwidth.  `us_per_layer`: one
    graph holds 2 * copies forwards (the copies in turn), as a model's captured decode
    step holds its layers, so no graph launch falls between two layers;
    `us_per_layer_one_graph_each`: one forward per graph, replayed round-robin, which adds
    a graph launch to every layer."""
    import torch

    import moe_synth as S
    layers = [moe_layer(sp, lay, layout)]
    for c in range(1, copies):
        layers.append(moe_layer(sp, clone_weights(lay), layout))
    res = {}
    s = torch.cuda.Stream()
    per_graph = 2 * copies
    stacked = max(1, replays // per_graph)
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
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs, stream=s):
            for j in range(per_graph):
                layers[j % copies].forward(x, *outs[j % copies])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(run, n):
            e0.record()
            for i in range(n):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1000.0

        for i in range(max(len(graphs), replays // 4)):  # untimed replays: steady clocks and queues
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        us_each = timed(lambda i: graphs[i % len(graphs)].replay(), replays) / replays
        for _ in range(max(2, stacked // 4)):
            gs.replay()
        torch.cuda.synchronize()
        us = timed(lambda i: gs.replay(), stacked) / (stacked * per_graph)
        w = alg_work(sp, T, outs[0][1], outs[0][3])
        gbs = w["bytes"] / (us * 1e-6) / 1e9
        gbs_each = w["bytes"] / (us_each * 1e-6) / 1e9
        res[f"T{T}"] = {"us_per_layer": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
                        "alg_bytes": w["bytes"], "touched_experts": w["touched"], "hbm_GBps": round(gbs, 1),
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "us_per_layer_one_graph_each": round(us_each, 2),
                        "hbm_frac_one_graph_each": round(gbs_each / HBM_PEAK_GBS, 4),
                        "routing": routing_report(layers[0], sp, x)}
        del graphs, gs
    return {"layer": name,
            "method": f"hipGraph replays over {copies} weight copies: {per_graph} forwards (the copies in turn) "
                      f"per graph, {stacked} replays; one_graph_each: one forward per graph, {replays} replays "
                      "round-robin (a graph launch per layer)",
            "points": res}


def decode_other(layout):
    """The other decode-sized layers the HBM target covers: Qwen3 INT4 at T=32 (4
    copies of its 0.31 GB of expert weights) and DeepSeek-V3 at T=1 and 16 (2 copies:
    one token already touches 0.8 GB), plus DeepSeek-V3 T=256 from its token sweep,
    and the OLMoE-shaped layer with FP8 experts (half the bf16 bytes) at T=1..64, with bf16
    activations and with FP8 activations (the streaming FP8 kernels on E4M3 codes up to T=32, the
    tiled FP8 MFMA kernels above)."""
    import torch

    import moe_synth as S
    out = {}
    for name, Ts, copies in (("qwen3_int4", (32,), 4), ("dsv3", (1, 16, 256), 2), ("olmoe_fp8", (1, 8, 32, 64), 4),
                              ("olmoe_fp8a8", (1, 8, 32, 64), 4)):
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


def prefill_point(sp, ml, x, steps, warmup):
    ms, per, outs, nl, wall = time_layer(ml, x, steps, warmup)
    T = x.shape[0]
    w = alg_work(sp, T, outs[1], outs[3])
    # flops per algorithmic byte; the ridge is the matrix peak over 8 TB/s (bf16 312.5, FP8 625)
    ai = w["flops"] / w["bytes"]
    peak = FP8_PEAK_TFLOPS if sp.expert == "fp8a8" else BF16_PEAK_TFLOPS
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "bound": "mfma" if ai >= peak / HBM_PEAK_GBS * 1e3 else "hbm",
            "flops_per_byte": round(ai, 1), "mfma_peak_tflops": peak,
            "hbm_frac_layer": round(w["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac_layer": round(w["flops"] / (ms * 1e-3) / 1e12 / peak, 4),
            "mfma_frac_gateup": round(w["gateup_flops"] / (per["gateup"] * 1e-3) / 1e12 / peak, 4),
            "per_launch_us": {n: round(v * 1e3, 2) for n, v in per.items()},
            "kept_pairs": w["kept"], "pairs": T * sp.k, "routing": routing_report(ml, sp, x)}, (ms, per, outs, nl,
                                                                                              wall, w)


def int4_drift(sp, lay, ml, x, layout):
    """Routing drift of the INT4 layer against its bf16 twin (the pre-quantisation weights
    rounded to bf16), in mean experts changed per token out of k.  In the layer itself the
    router is bf16 and sees the same x, so its picks cannot move; what moves is the
    residual stream after the layer, x + out, that the next layer's router sees.  That is
    measured with this layer's router standing in for the next one's."""
    import torch

    import moe_synth as S
    wg, wu, wd = S.make_bf16_twin(sp, device="cuda")
    twin_sp = sp.replace(expert="bf16")
    twin = moe_layer(twin_sp, S.Layer(twin_sp, lay.w_router, lay.logit_bias, lay.select_bias, wg, wu, wd), layout)
    out_q, idx_q, _, _ = ml.forward(x)
    out_b, idx_b, _, _ = twin.forward(x)

    def swaps(a, b):
        same = (a[:, :, None] == b[:, None, :]).any(2).sum(1)
        return float((sp.k - same).float().mean())

    nxt_q = ml.route((x.float() + out_q.float()).to(x.dtype), want_scores=False)[0]
    nxt_b = twin.route((x.float() + out_b.float()).to(x.dtype), want_scores=False)[0]
    rel = float(((out_q.float() - out_b.float()).norm() / out_b.float().norm()))
    del twin, wg, wu, wd
    torch.cuda.empty_cache()
    return {"tokens": x.shape[0], "k": sp.k, "swaps_per_token_this_layer": swaps(idx_q, idx_b),
            "swaps_per_token_next_router": swaps(nxt_q, nxt_b), "out_rel_l2_vs_bf16_twin": round(rel, 5)}


def prefill_sweep(layout, steps=20, warmup=3):
    """The other prefill layers: DeepSeek-V2-Lite T=8192 (dropless and C=1.25), the
    DeepSeek-V3 token-sweep step T=4096, the INT4 layer at T=4096 (with its routing drift),
    FP8 experts (OLMoE-shaped T=4096, DeepSeek-V2-Lite-shaped T=8192 with FP8 shared
    experts), and FP8 experts with FP8 activations (OLMoE-shaped T=4096, DeepSeek-V2-Lite-shaped
    T=8192 with its two shared experts, DeepSeek-V3-shaped T=16384): useful-flop fraction of the matrix peak the layer multiplies at (bf16, or FP8
    for FP8 activations; `mfma_peak_tflops`) of the whole layer and of its gate/up launch
    (with FP8 activations the gate/up and down figures include the row quantisation ahead of
    each GEMM)."""
    import torch

    import moe_synth as S
    res = {}
    for name, Ts in (("dsv2_lite", (8192,)), ("dsv2_lite_cap", (8192,)), ("dsv3", (4096,)), ("qwen3_int4", (4096,)),
                     ("olmoe_fp8", (4096,)), ("dsv2_lite_fp8", (8192,)), ("olmoe_fp8a8", (4096,)),
                     ("dsv2_lite_fp8a8", (8192,)), ("dsv3_fp8a8", (16384,))):
        sp = S.SPECS[name]
        lay = S.make_layer(sp, device="cuda")
        ml = moe_layer(sp, lay, layout)
        for T in Ts:
            x = S.make_tokens(sp, T, device="cuda")
            res[f"{name}_T{T}"] = prefill_point(sp, ml, x, steps, warmup)[0]
            if sp.expert == "int4":
                res[f"{name}_T{T}"]["drift"] = int4_drift(sp, lay, ml, x, layout)
            del x
        del ml, lay
        torch.cuda.empty_cache()
    return {"method": f"eager, {steps} timed forwards after {warmup}; useful flops only (dropped pairs and tile "
                      "padding excluded)", "points": res}


def ep_shard(sp, lay, x, idx, layout, n_gpus=8, steps=10, warmup=3):
    """One GPU's share of the layer under expert parallelism over n_gpus GPUs (a design the
    library does not run across GPUs; this measures its per-GPU kernel work at the real shape):
    experts 0 .. E/n_gpus - 1 of the layer, fed the rows that the routing of all T tokens sends
    to them, as a dispatch all-to-all would deliver them.  Each received row is one local token
    with its one local expert and gate 1, run as the route-replay forward (permutation, expert
    GEMMs, combine into received-row order); the shared expert, which each GPU would run on its
    own T / n_gpus tokens, is left out.  Eager forwards timed between two events."""
    import torch

    import moe_synth as S
    E_loc = sp.E // n_gpus
    t_idx, j_idx = (idx < E_loc).nonzero(as_tuple=True)
    x_recv = x[t_idx].contiguous()
    idx_loc = idx[t_idx, j_idx].to(torch.int32).view(-1, 1).contiguous()
    gates = torch.ones(idx_loc.shape, dtype=torch.float32, device=x.device)
    R = int(x_recv.shape[0])
    sp_loc = sp.replace(name=f"{sp.name}_ep{n_gpus}_shard0", E=E_loc, k=1, n_shared=0, ffn_shared=0,
                        score="softmax", renorm=False, gate_scale=1.0, logit_bias_std=0.0, select_bias_std=0.0)
    lay_loc = S.Layer(sp_loc, lay.w_router[:E_loc].contiguous(), None, None, lay.w_gate[:E_loc], lay.w_up[:E_loc],
                      lay.w_down[:E_loc])
    ml = moe_layer(sp_loc, lay_loc, layout)
    for _ in range(warmup):
        ml.forward_with_routes(x_recv, idx_loc, gates)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ml.forward_with_routes(x_recv, idx_loc, gates)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 6.0 * sp.d * sp.ffn * R
    out = {"n_gpus": n_gpus, "local_experts": E_loc, "rows_received": R,
           "rows_per_gpu_if_balanced": int(idx.numel()) // n_gpus, "ms_per_step": round(ms, 4),
           "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "method": f"route-replay forward of experts 0..{E_loc - 1} on the rows the routing sends them; "
                     f"eager, {steps} timed after {warmup}; shared expert not included"}
    del ml, lay_loc, x_recv
    torch.cuda.empty_cache()
    return out


def roofline_of(sp, T, w, per, workload):
    t_gu = per["gateup"] * 1e-3
    achieved = w["gateup_flops"] / t_gu / 1e12
    kernel = GATEUP_KERNELS[TRAFFIC_WORKLOADS[workload][2]][1] if workload in TRAFFIC_WORKLOADS else "gate/up"
    return {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_record(workload), "alg_bytes_per_launch": gateup_alg_bytes(sp, T, w),
            "avg_launch_us": round(per["gateup"] * 1e3, 2), "alg_flops_per_launch": w["gateup_flops"]}


def main():
    args = parse()
    if args.traffic_record:
        spec, T, _ = TRAFFIC_WORKLOADS[args.traffic_workload]
        cmds = [f"rocprofv3 --pmc {c} --kernel-include-regex {rx} --output-format csv -d <out> -o pmc -- "
                f"python3 bench.py {a}"
                for rx, a in (("ffn_tiled", f"--profile-layer {spec} --T {T} --steps 3 --warmup 1"),
                              ("copyBuffer", "--copy-probe"))
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        write_traffic_record(args.traffic_workload, *args.traffic_record, commands=cmds)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the layer on one GPU only (asked for {max(args.gpus, world)}): the path has no "
              "multi-GPU mode (expert-parallel sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_synth as S

    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.memory_probe:
        print(json.dumps(memory_probe()), flush=True)
        return
    if args.profile_layer:
        psp = S.SPECS[args.profile_layer]
        play = S.make_layer(psp, device="cuda")
        ml = moe_layer(psp, play, args.layout)
        x = S.make_tokens(psp, args.T, device="cuda")
        ms = time_layer(ml, x, args.steps, args.warmup)[0]
        print(json.dumps({"layer": args.profile_layer, "T": args.T, "ms_per_forward": round(ms, 4)}), flush=True)
        return
    if args.decode_only:
        sp = S.SPECS["olmoe"]
        lay = S.make_layer(sp, device="cuda")
        print(json.dumps(decode_sweep(sp, lay, args.layout)), flush=True)
        del lay
        torch.cuda.empty_cache()
        print(json.dumps(decode_other(args.layout)), flush=True)
        return

    # ---- headline: the DeepSeek-V3-shaped layer at T tokens
    sp = S.SPECS["dsv3"]
    T = args.T
    workload = f"dsv3_T{T}"
    lay = S.make_layer(sp, device="cuda")
    x = S.make_tokens(sp, T, device="cuda")
    ml = moe_layer(sp, lay, args.layout)
    K = args.steps
    head, (ms_step, per, outs, nl, wall, w) = prefill_point(sp, ml, x, K, args.warmup)
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
        "config": {"workload": f"deepseek_v3_layer_T{T}", "T": T, "d": sp.d, "E": sp.E, "k": sp.k, "ffn": sp.ffn,
                   "n_shared": sp.n_shared, "ffn_shared": sp.ffn_shared, "launches_per_layer": nl,
                   "weight_layout": args.layout},
        "roofline": roofline_of(sp, T, w, per, workload),
        "layer": {"per_launch_us": head["per_launch_us"], "alg_flops": w["flops"], "alg_bytes": w["bytes"],
                  "mfma_frac": head["mfma_frac_layer"], "kept_pairs": w["kept"], "touched_experts": w["touched"],
                  "wall_s_timed": round(wall, 3)},
        "routing": {workload: head["routing"]},
    }
    line["ep8_shard"] = ep_shard(sp, lay, x, outs[1], args.layout)
    del ml, outs
    torch.cuda.empty_cache()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(sp, lay, x, n_ffn=1024)
    del lay, x
    torch.cuda.empty_cache()

    # ---- the OLMoE-shaped layer at T=4096 (a prefill-sized sub-key) and its decode sizes
    osp = S.SPECS["olmoe"]
    olay = S.make_layer(osp, device="cuda")
    ox = S.make_tokens(osp, 4096, device="cuda")
    oml = moe_layer(osp, olay, args.layout)
    opt, (oms, oper, oouts, _, _, ow) = prefill_point(osp, oml, ox, K, args.warmup)
    opt["roofline"] = roofline_of(osp, 4096, ow, oper, "olmoe_T4096")
    line["olmoe_T4096"] = opt
    del oml, oouts, ox
    if not args.no_decode:
        line["decode"] = decode_sweep(osp, olay, args.layout)
        del olay
        torch.cuda.empty_cache()
        line["decode_other"] = decode_other(args.layout)
    else:
        del olay
    torch.cuda.empty_cache()
    if not args.no_prefill:
        line["prefill"] = prefill_sweep(args.layout)
    line["memory_probe"] = memory_probe()
    line["pages_context"] = PAGES_CONTEXT
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
