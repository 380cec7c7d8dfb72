"""Benchmark of the Beam MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
python bench.py --workload NAME --sweep 16,64,256,... [--steps K]   (one line per T)

A step is one full `beam_moe_forward` (router, permutation, gate/up GEMM with SwiGLU,
down GEMM, combine) -- or `beam_moe_sublayer_forward` for the sublayer workload, and
`beam_dense_forward` for the dense-MLP workloads -- over one batch of seeded synthetic
Beam-shaped inputs already resident in HBM.  Prints ONE JSON line on stdout; progress
goes to stderr.

Default workload: the Beam-shaped layer (hidden 5120, 256 experts in 8 groups of 32,
top-4 groups, top-8, SwiGLU intermediate 2560, BF16 experts) at 32768 tokens with skewed
routing (Zipf(1.1) logit offsets over a random expert permutation), the largest
configuration on one GPU, where the expert GEMMs are bound by the matrix cores.  The
same run times the decode batch (16 tokens, x RMS-normalised, the same weights), which
streams the weights of every routed expert from HBM, and carries it in `extra`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % of MI355X MFMA peak (prefill) / HBM GB/s (decode)"
HBM_PEAK_GBS = 8000.0
# dense peaks: bf16, fp8, fp32 (vector); MXFP4 weights meet E4M3 activations, an FP8 x FP4
# product priced at the FP8 rate
MFMA_PEAK_TFLOPS = {1: 2500.0, 2: 5000.0, 3: 5000.0, 0: 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="beam_skewed_t32768")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode-batch measurement carried in `extra` of the default line")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=16)
    p.add_argument("--sweep", default="", metavar="T1,T2,...",
                   help="time the workload's layer at each token count (prefixes of its tokens); "
                        "one JSON line per count")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run 3 plain device copies of MIB MiB (reference for HBM byte counters)")
    return p.parse_args()


def calibrate_copy(mib: int):
    """Plain device-to-device copies of a known size: the profiler's FETCH_SIZE /
    WRITE_SIZE for these dispatches, divided into the known bytes, give the factor that
    turns those counters into bytes for the layer's kernels."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)


class Layer:
    """Device copies of one workload's weights (inputs resident in HBM) and a step
    function for any token count up to the workload's T."""

    def __init__(self, w, inp):
        import torch
        import sparse_mixture_experts_group_amd as bm
        self.bm, self.w, self.inp = bm, w, inp
        self.dev = dev = torch.device("cuda:0")

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        self.x_all = up(inp.x)
        self.wr = up(inp.w_router) if inp.w_router is not None else None
        self.w13, self.w2 = up(inp.w13), up(inp.w2)
        self.s13 = up(inp.w13_scale) if inp.w13_scale is not None else None
        self.s2 = up(inp.w2_scale) if inp.w2_scale is not None else None
        self.bias = up(inp.logit_bias) if inp.logit_bias is not None else None
        kind = bm.BEAM_FP8_SCALES_POW2 if w.fp8_scales == "pow2" else bm.BEAM_FP8_SCALES_FP32
        if w.dense:
            self.cfg = bm.make_dense_config(hidden=w.H, inter=w.I, act_dtype=w.act_dtype,
                                            weight_dtype=w.weight_dtype, fp8_block=w.fp8_block, norm_eps=w.norm_eps,
                                            fp8_scale_kind=kind)
        else:
            self.cfg = bm.make_config(hidden=w.H, inter=w.I, n_experts=w.E, n_groups=w.G, topk_groups=w.Kg,
                                      topk=w.K, routed_scale=w.alpha, act_dtype=w.act_dtype,
                                      weight_dtype=w.weight_dtype, fp8_block=w.fp8_block, norm_eps=w.norm_eps,
                                      fp8_scale_kind=kind)

    def measure(self, T: int, steps: int, warmup: int, x_rows=None, bias="layer") -> dict:
        """Time `steps` forwards over the first T tokens (after `warmup` untimed ones):
        step time from HIP events and the wall clock, the gate/up GEMM's duration from
        events the library records around it, then the other kernels in separate passes.
        x_rows: other activations [T, H] (device) in place of the workload's; bias: the
        logit offsets to use ("layer": the workload's)."""
        import torch
        bm, w = self.bm, self.w
        x = (self.x_all[:T] if x_rows is None else x_rows).contiguous()
        lbias = self.bias if isinstance(bias, str) else bias
        ws = (bm.alloc_dense_workspace if w.dense else bm.alloc_workspace)(self.cfg, T, self.dev)
        ids = torch.empty((T, w.K), dtype=torch.int32, device=self.dev)
        wts = torch.empty((T, w.K), dtype=torch.float32, device=self.dev)
        y = torch.empty_like(x)
        h = x.clone()      # the sublayer updates the residual stream in place, step after step

        def step():
            if w.dense and w.sublayer:
                bm.beam_dense_sublayer_forward(self.cfg, h, w.step_k, self.w13, self.w2, w13_scale=self.s13,
                                               w2_scale=self.s2, ws=ws)
            elif w.dense:
                bm.beam_dense_forward(self.cfg, x, self.w13, self.w2, w13_scale=self.s13, w2_scale=self.s2, y=y,
                                      ws=ws)
            elif w.sublayer:
                bm.beam_moe_sublayer_forward(self.cfg, h, w.step_k, self.wr, self.w13, self.w2,
                                             logit_bias=lbias, w13_scale=self.s13, w2_scale=self.s2,
                                             ids=ids, weights=wts, ws=ws)
            else:
                bm.beam_moe_forward(self.cfg, x, self.wr, self.w13, self.w2, logit_bias=lbias,
                                    w13_scale=self.s13, w2_scale=self.s2, y=y, ids=ids, weights=wts, ws=ws)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        timer = bm.KernelTimer(bm.BEAM_KERNEL_GATE_UP, steps)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        with timer:
            ev0.record()
            for _ in range(steps):
                step()
            ev1.record()
            torch.cuda.synchronize()
        wall1 = time.perf_counter()
        ms_gpu = ev0.elapsed_time(ev1) / steps
        ms_wall = (wall1 - wall0) * 1e3 / steps
        kernel_ms = {"gate_up": round(float(np.mean(timer.times_ms())), 4)}
        # per-kernel times (separate passes after the timed region)
        others = [("router_logits", bm.BEAM_KERNEL_ROUTER_LOGITS), ("down", bm.BEAM_KERNEL_DOWN),
                  ("combine", bm.BEAM_KERNEL_COMBINE)]
        if w.dense:             # no router; the combine kernel only inside the sublayer
            others = [o for o in others if o[0] == "down" or (o[0] == "combine" and w.sublayer)]
        for name, kid in others:
            n = min(steps, 3)
            kt = bm.KernelTimer(kid, n)
            with kt:
                for _ in range(n):
                    step()
                torch.cuda.synchronize()
            kernel_ms[name] = round(float(np.mean(kt.times_ms())), 4)
        if w.dense:
            return {"ms_gpu": ms_gpu, "ms_wall": ms_wall, "ms_per_step": max(ms_gpu, ms_wall),
                    "kernel_ms": kernel_ms, "n_active": 1, "max_rows": T}
        ids_np = ids.cpu().numpy()
        return {"ms_gpu": ms_gpu, "ms_wall": ms_wall, "ms_per_step": max(ms_gpu, ms_wall),
                "kernel_ms": kernel_ms, "n_active": int(np.unique(ids_np).size),
                "max_rows": int(np.bincount(ids_np.reshape(-1), minlength=w.E).max())}


def gate_up_roofline(w, T: int, n_active: int, gate_up_ms: float) -> dict:
    """Roofline of the grouped gate/up GEMM: algorithmic bytes (routed experts' gate/up
    weights, scales, x, the SwiGLU output) and flops per launch over its duration; the
    bound is whichever of the HBM and MFMA times is larger."""
    from beam_inputs import DT_BF16, DT_FP8, DT_F32, DT_MXFP4
    P = T * w.K
    wbytes = {DT_F32: 4, DT_BF16: 2, DT_FP8: 1, DT_MXFP4: 0.5}[w.weight_dtype]
    abytes = {DT_F32: 4, DT_BF16: 2, DT_FP8: 1, DT_MXFP4: 1}[w.weight_dtype]   # the GEMM's A operand
    gate_up_weight_bytes = n_active * 2 * w.I * w.H * wbytes
    if w.weight_dtype == DT_FP8:
        gate_up_weight_bytes += n_active * (2 * w.I // 128) * (w.H // 128) * 4
    if w.weight_dtype == DT_MXFP4:
        gate_up_weight_bytes += n_active * 2 * w.I * (w.H // 32)
    gate_up_bytes = gate_up_weight_bytes + T * w.H * abytes + P * w.I * 2
    gate_up_flops = 2.0 * P * w.H * 2 * w.I
    peak_tf = MFMA_PEAK_TFLOPS[w.weight_dtype]
    t_hbm = gate_up_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = gate_up_flops / (peak_tf * 1e12)
    if t_hbm >= t_mfma:
        achieved = gate_up_bytes / (gate_up_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = gate_up_flops / (gate_up_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4)}
    roof.update({"kernel": "grouped gate/up GEMM + SwiGLU", "kernel_ms": round(gate_up_ms, 4),
                 "algorithmic_bytes": int(gate_up_bytes), "algorithmic_flops": gate_up_flops})
    return roof


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer is built and timed on a single MI355X; "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    from beam_inputs import WORKLOADS, make_inputs, DT_F32, DTYPE_NAMES

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = WORKLOADS[args.workload]
    if args.sweep:
        ts = [int(t) for t in args.sweep.split(",")]
        w = w.with_T(max(ts))
    t0 = time.time()
    log(f"[bench] generating inputs for {w.name} (T={w.T}) ...")
    inp = make_inputs(w)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; uploading")
    layer = Layer(w, inp)

    if args.sweep:
        # one JSON line per token count (batch sizes between decode and prefill)
        for T in ts:
            r = layer.measure(T, args.steps, args.warmup)
            roof = gate_up_roofline(w, T, r["n_active"], r["kernel_ms"]["gate_up"])
            wbytes = {0: 4, 1: 2, 2: 1, 3: 0.5}[w.weight_dtype]
            layer_wbytes = r["n_active"] * 3 * w.I * w.H * wbytes
            print(json.dumps({"sweep": w.name, "T": T, "ms_per_step": round(r["ms_per_step"], 4),
                              "tokens_per_s": round(T / (r["ms_per_step"] / 1e3), 1),
                              "distinct_experts": r["n_active"], "max_rows_per_expert": r["max_rows"],
                              "layer_weight_gbs": round(layer_wbytes / (r["ms_per_step"] / 1e3) / 1e9, 1),
                              "gate_up_roofline": {k: roof[k] for k in ("bound", "achieved", "unit", "frac")},
                              "kernel_ms": r["kernel_ms"]}), flush=True)
        return

    K = args.steps
    r = layer.measure(w.T, K, args.warmup)
    ms_per_step = r["ms_per_step"]
    tokens_per_s = w.T / (ms_per_step / 1e3)
    roof = gate_up_roofline(w, w.T, r["n_active"], r["kernel_ms"]["gate_up"])
    roof["traffic"] = measured_traffic(w.name)

    # ---- whole-layer figures ----
    P = w.T * w.K
    wbytes = {0: 4, 1: 2, 2: 1, 3: 0.5}[w.weight_dtype]
    layer_flops = 2.0 * P * w.H * 3 * w.I + (0.0 if w.dense else 2.0 * w.T * w.H * w.E)
    layer_wbytes = r["n_active"] * 3 * w.I * w.H * wbytes
    extra = {"layer_tflops": round(layer_flops / (ms_per_step / 1e3) / 1e12, 2),
             "layer_weight_gbs": round(layer_wbytes / (ms_per_step / 1e3) / 1e9, 1),
             "distinct_experts": r["n_active"], "max_rows_per_expert": r["max_rows"],
             "ms_gpu_events": round(r["ms_gpu"], 4), "ms_wall": round(r["ms_wall"], 4),
             "kernel_ms": r["kernel_ms"]}

    # ---- the decode batch on the same weights (the HBM-bound half of the metric) ----
    wd = WORKLOADS["beam_decode_t16"]
    same_layer = (not w.dense and (w.H, w.I, w.E, w.G, w.Kg, w.K, w.weight_dtype, w.seed) ==
                  (wd.H, wd.I, wd.E, wd.G, wd.Kg, wd.K, wd.weight_dtype, wd.seed))
    if not args.no_decode and same_layer and w.name != wd.name:
        extra["decode_t16"] = decode_line(layer, wd, K, args.warmup)

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_sample_tokens)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAMES[w.weight_dtype] if w.weight_dtype != DT_F32 else "f32",
        "data": "synthetic (seeded Philox normals, Beam-shaped, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "hidden": w.H, "intermediate": w.I, "experts": w.E,
                   "groups": w.G, "topk_groups": w.Kg, "topk": w.K, "routed_scale": w.alpha,
                   "weights": DTYPE_NAMES[w.weight_dtype], "sublayer": w.sublayer, "dense_mlp": w.dense,
                   "zipf_s": w.zipf_s, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(out), flush=True)


def decode_line(layer, wd, steps: int, warmup: int) -> dict:
    """The decode batch (16 tokens, x RMS-normalised, no logit offsets) through the
    layer's weights, timed like the main line: step time, gate/up GEMM time and its HBM
    roofline fraction."""
    import torch
    from beam_inputs import token_inputs, to_bf16_bits
    xd = torch.from_numpy(to_bf16_bits(token_inputs(wd)).view(np.int16)).to(layer.dev).view(torch.bfloat16)
    log(f"[bench] decode batch T={wd.T} on the same weights ...")
    r = layer.measure(wd.T, max(steps, 20), warmup, x_rows=xd, bias=None)
    roof = gate_up_roofline(wd, wd.T, r["n_active"], r["kernel_ms"]["gate_up"])
    roof["traffic"] = measured_traffic(wd.name)
    layer_wbytes = r["n_active"] * 3 * wd.I * wd.H * 2
    return {"workload": wd.name, "T": wd.T, "ms_per_step": round(r["ms_per_step"], 4),
            "tokens_per_s": round(wd.T / (r["ms_per_step"] / 1e3), 1), "distinct_experts": r["n_active"],
            "layer_weight_gbs": round(layer_wbytes / (r["ms_per_step"] / 1e3) / 1e9, 1),
            "layer_hbm_frac": round(layer_wbytes / (r["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": roof, "kernel_ms": r["kernel_ms"]}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    passes (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a plain copy of
    known size), or None when there is no record for this workload or a source of the
    kernel has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec:
        return None
    srcs = rec.get("sources", [rec.get("source")])
    shas = rec.get("sources_sha256", [rec.get("source_sha256")])
    for name, sha in zip(srcs, shas):
        src = os.path.join(ROOT, name)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != sha:
            return None
    return rec["traffic_bytes_per_launch"]


def cpu_baseline(w, inp, n_tok):
    """Time the CPU oracle (as it stands) on the first n_tok tokens of the workload:
    full FP32 routing of those tokens plus their float64 expert MLPs and combine."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    n = min(n_tok, w.T)
    if w.act_dtype == 0:
        x32 = inp.x[:n]
    else:
        x32 = oracle.bf16_to_f32(inp.x[:n])
    bank = oracle.ExpertBank(inp.w13, inp.w2, {0: "f32", 1: "bf16", 2: "fp8_e4m3", 3: "mxfp4"}[w.weight_dtype],
                             inp.w13_scale, inp.w2_scale, w.fp8_block)
    log(f"[bench] timing the CPU oracle on {n} tokens ...")

    def run_once():
        if w.dense and w.sublayer:
            oracle.dense_sublayer_forward(x32, None, None, w.step_k, w.norm_eps, bank)
        elif w.dense:
            oracle.dense_forward(x32, bank)
        elif w.sublayer:
            oracle.sublayer_forward(x32, None, None, w.step_k, w.norm_eps, inp.w_router, inp.logit_bias, bank,
                                    w.G, w.Kg, w.K, w.alpha)
        else:
            oracle.moe_forward(x32, inp.w_router, inp.logit_bias, bank, w.G, w.Kg, w.K, w.alpha)

    # repeated until about 10 s of CPU work (at most 8 runs), averaged per run
    runs = 0
    t0 = time.perf_counter()
    while True:
        run_once()
        runs += 1
        if time.perf_counter() - t0 >= 10.0 or runs >= 8:
            break
    total = time.perf_counter() - t0
    dt = total / runs
    log(f"[bench] CPU oracle: {runs} runs, {dt:.2f}s each")
    what = "float64 dense SwiGLU MLP" if w.dense else "FP32 routing + float64 expert MLPs and combine"
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": int(max(oracle.num_threads(), blas)),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "kind": "oracle", "seconds": round(total, 2), "runs": runs,
            "sample": f"first {n} tokens of {w.name}, {runs} runs: {what}"}


if __name__ == "__main__":
    main()
