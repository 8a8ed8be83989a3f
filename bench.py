#!/usr/bin/env python3
"""Benchmark of the fused MoE forward on one MI355X (gfx950).

One step = one moe_forward over the whole batch: router -> align ->
[fp8 quant] -> grouped GEMM W13 + SiLU*up -> grouped GEMM W2 -> top-k
weight-and-reduce, on seeded synthetic inputs already resident in HBM.
Prints one JSON line.  Default workload: the DeepSeek-V3-like layer with
grouped sigmoid routing (M 4096, H 7168, I 2048, E 256, top-8, bf16), the
largest configuration that fits one GPU.

The `roofline` object covers the dominant kernel (the W13 GEMM).  Its
algorithmic bytes per launch are the weights of the experts that received
rows (+ their biases and scales) plus the activation rows read once; its
output z is an intermediate of this implementation, reported separately as
`materialised_bytes`.  `achieved` divides the bytes (or, where the kernel is
MFMA-bound, 2 x rows x H x 2I FLOPs) by the kernel's average duration, timed
with HIP events recorded on the launch stream around that kernel in every
timed step; `profile_avg_ms` is the same kernel's average from the committed
rocprofv3 summary when it was taken on the current GEMM sources.
`cpu_baseline` times the CPU oracle (test infrastructure, untuned) on a
bounded token sample of the same workload on all of this host's cores.
"""
import argparse
import dataclasses
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE fwd tokens/s + active TFLOP/s (or HBM GB/s), % of roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}
# the largest configuration that fits one GPU: the headline
DEFAULT_WORKLOAD = "deepseek_grouped_sigmoid_bf16"
# the other problem configurations, summarised in the default line
OTHER_CONFIGS = ("tiny_f32", "mixtral_prefill_bf16", "decode_e128_bf16", "batched_fp8_skewed")
OTHER_STEPS, OTHER_WARMUP = 20, 5


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens (or batched rows) the CPU oracle leg computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time the default workload only (no per-configuration summaries)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 5 times (the "
                         "reference point for scaling HBM byte counters), then exit")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.handles.append(e.value)
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                          ctypes.c_void_p(b))
        if rc != 0:
            self.hip.hipGetLastError()      # do not leave the error pending for later calls
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for h in self.handles:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.handles = []


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported: the fused MoE forward here runs on a single device and no multi-GPU "
              "path exists to time.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    from mixture_experts_ffn_router_amd import binding as B
    from mixture_experts_ffn_router_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel(), "launches": 5}), flush=True)
        return
    cfg = W.BY_NAME[args.workload]
    res, inp, info = measure(cfg, args.steps, args.warmup, args.seed, time_plain=True)

    # ---- the other problem configurations (default run only):
    # one summary per workload in the same line, so that every configuration's
    # throughput and roofline fraction is measured by the same invocation
    if args.workload == DEFAULT_WORKLOAD and not args.no_other_configs:
        res["configs"] = {}
        for name in OTHER_CONFIGS:
            torch.cuda.empty_cache()
            r, _, _ = measure(W.BY_NAME[name], OTHER_STEPS, OTHER_WARMUP, None, time_plain=False)
            res["configs"][name] = summary(r)
        torch.cuda.empty_cache()

    # ---- CPU oracle leg (rank 0, N = 1 only)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, info, args.cpu_sample)
    print(json.dumps(res), flush=True)


def summary(r):
    """The figures of one workload's measurement kept in the headline line."""
    roof = r["roofline"]
    return {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["value"], "steps": r["steps"],
            "dtype": r["dtype"], "stage_ms": r["stage_ms"],
            "gemm1": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                           "kernel")},
            "path_roofline_frac": r["path_roofline"]["frac"],
            "active_tflops": r["active_tflops"], "hbm_gbs_path": r["hbm_gbs_path"]}


def measure(cfg, steps, warmup, seed, time_plain):
    """Times `steps` forwards of workload `cfg` after `warmup` untimed ones;
    returns (result dict, inputs, workspace info)."""
    import numpy as np
    import torch
    from mixture_experts_ffn_router_amd import binding as B
    from mixture_experts_ffn_router_amd import workloads as W

    dev = torch.device("cuda:0")
    seed = seed if seed is not None else (
        1000 + W.CONFIGS.index(cfg) if cfg in W.CONFIGS else 1100 + W.EXTRA.index(cfg))
    print(f"[bench] {cfg.name}: generating inputs (seed {seed})", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    batched = cfg.fmt == "batched"

    # ---- problem and arguments (marshalling only)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    out_dt = tdt[cfg.out_dtype]
    wq_bits = {"u8": 8, "u4": 4}.get(cfg.weight, 0)           # WNA16 weight codes
    w_code = {8: B.MOE_U8, 4: B.MOE_U4}[wq_bits] if wq_bits else B._dtype_code(inp["w13"])
    # block-wise fp8 scales and WNA16 codes run on packed weights only
    layout0 = B.MOE_W_PACKED if (cfg.fp8_block or wq_bits) else B.MOE_W_PLAIN
    if batched:
        hidden = inp["hidden"]
        prob = B.Problem(M=cfg.M, H=cfg.H, I=cfg.I, E=cfg.E, top_k=cfg.top_k,
                         fmt=B.MOE_FMT_BATCHED, max_tokens=inp["max_tokens"],
                         act_dtype=B._dtype_code(hidden), w_dtype=w_code,
                         out_dtype=B._dtype_code(torch.empty(0, dtype=out_dt)),
                         routing=B.MOE_ROUTE_PRECOMPUTED, fp8_block=cfg.fp8_block,
                         w_layout=layout0)
        out = torch.empty(cfg.E, inp["max_tokens"], cfg.H, dtype=out_dt, device=dev)
        cargs = B.make_args(hidden, inp["w13"], inp["w2"], out,
                            expert_num_tokens=inp["expert_num_tokens"],
                            w13_scale=inp.get("w13_scale"), w2_scale=inp.get("w2_scale"),
                            w13_zero=inp.get("w13_zero"), w2_zero=inp.get("w2_zero"))
    else:
        hidden = inp["hidden"]
        emap = inp.get("expert_map")
        E_local = inp["w13"].shape[0]
        prob = B.Problem(M=cfg.M, H=cfg.H, I=cfg.I, E=E_local, top_k=cfg.top_k,
                         global_experts=0 if emap is None else cfg.E,
                         act_dtype=B._dtype_code(hidden), w_dtype=w_code,
                         out_dtype=B._dtype_code(torch.empty(0, dtype=out_dt)),
                         logits_dtype=B._dtype_code(inp["logits"]),
                         routing=B.MOE_ROUTE_SIGMOID if cfg.scoring == "sigmoid"
                         else B.MOE_ROUTE_SOFTMAX,
                         renormalize=cfg.renormalize, group_count=cfg.group_count,
                         k_group=cfg.k_group, group_select_mode=cfg.group_select_mode,
                         routed_scaling_factor=cfg.routed_scaling_factor,
                         has_w13_bias=inp["w13_bias"] is not None,
                         has_w2_bias=inp["w2_bias"] is not None, fp8_block=cfg.fp8_block,
                         w_layout=layout0)
        out = torch.empty(cfg.M, cfg.H, dtype=out_dt, device=dev)
        cargs = B.make_args(hidden, inp["w13"], inp["w2"], out, router_logits=inp["logits"],
                            w13_bias=inp["w13_bias"], w2_bias=inp["w2_bias"],
                            w13_scale=inp.get("w13_scale"), w2_scale=inp.get("w2_scale"),
                            expert_map=emap, w13_zero=inp.get("w13_zero"),
                            w2_zero=inp.get("w2_zero"))
    # one workspace for both weight layouts (their tile choices, and so their
    # workspace layouts, may differ); `info` describes the packed (timed) one
    ws, info = B.allocate_workspace(prob, dev)
    if cfg.weight in ("bf16", "fp8", "u8", "u4") and layout0 == B.MOE_W_PLAIN:
        info = B.moe_workspace_shapes(dataclasses.replace(prob, w_layout=B.MOE_W_PACKED).c())
        if int(info.bytes) > ws.numel():
            ws = torch.empty(int(info.bytes), dtype=torch.uint8, device=dev)
    stream = B.current_stream_handle(dev)
    hip = HipEvents()
    rec = hip.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    nst = len(B.STAGES)

    # ---- weights: bf16 expert weights are re-laid out once, as at model load
    # (moe_pack_weights); the plain layout is timed too, for reference
    plain_prob, plain_args = prob.c(), cargs
    pack_ms = None
    if cfg.weight in ("bf16", "fp8", "u8", "u4"):
        ev0, ev1 = hip.create(), hip.create()
        rec(ctypes.c_void_p(ev0), ctypes.c_void_p(stream))
        pw = B.pack_weights(inp["w13"], inp["w2"], wq_bits=wq_bits)
        rec(ctypes.c_void_p(ev1), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        pack_ms = hip.elapsed_ms(ev0, ev1)
        prob.w_layout = B.MOE_W_PACKED
        cargs = B.moe_args.from_buffer_copy(cargs)
        cargs.w13, cargs.w2 = pw.w13.data_ptr(), pw.w2.data_ptr()
    cprob = prob.c()

    def run_steps(p, a, n):
        for _ in range(n):
            B.moe_forward(p, a, ws.data_ptr(), ws.numel(), stream)

    # ---- warmup
    run_steps(cprob, cargs, warmup)
    torch.cuda.synchronize()

    # ---- timed steps: K back-to-back forwards between two synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(cprob, cargs, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps

    # ---- the same steps again with HIP events on the launch stream around
    # every step and every kernel stage (per-kernel durations, roofline)
    step_ev = [(hip.create(), hip.create()) for _ in range(steps)]
    stage_ev = [[hip.create() for _ in range(2 * nst)] for _ in range(steps)]
    for k in range(steps):
        rec(ctypes.c_void_p(step_ev[k][0]), ctypes.c_void_p(stream))
        B.moe_forward_timed(cprob, cargs, ws.data_ptr(), ws.numel(), stream, stage_ev[k])
        rec(ctypes.c_void_p(step_ev[k][1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(a, b) for a, b in step_ev]
    stage_ms = {}
    for s, name in enumerate(B.STAGES):
        try:
            vals = [hip.elapsed_ms(ev[2 * s], ev[2 * s + 1]) for ev in stage_ev]
        except RuntimeError:
            continue            # stage not run for this problem
        stage_ms[name] = float(np.mean(vals))

    # ---- plain weight layout, for reference (same steps, same clock)
    plain_ms = None
    if time_plain and pack_ms is not None and layout0 == B.MOE_W_PLAIN:   # some run packed only
        run_steps(plain_prob, plain_args, 2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(plain_prob, plain_args, steps)
        torch.cuda.synchronize()
        plain_ms = (time.perf_counter() - t0) * 1e3 / steps
    hip.close()

    # ---- accounting
    if batched:
        counts = inp["expert_num_tokens"].cpu().numpy()
        valid_rows = int(counts.sum())
    else:
        off = info.off_expert_counts
        counts = ws[off:off + 4 * prob.E].view(torch.int32).cpu().numpy()
        valid_rows = int(counts.sum())          # M * top_k, or this shard's routed rows
    active = int((counts > 0).sum())
    wes = {"f32": 4, "bf16": 2, "fp8": 1, "u8": 1, "u4": 0.5}[cfg.weight]
    aes = {"f32": 4, "bf16": 2}[cfg.act]
    oes = {"f32": 4, "bf16": 2}[cfg.out_dtype]
    zes = 1 if cfg.weight == "fp8" else aes
    w13_b = int(active * cfg.H * 2 * cfg.I * wes)
    w2_b = int(active * cfg.I * cfg.H * wes)
    if wq_bits:                             # group scales (+ zero points) per 128 K rows
        ng = lambda k: -(-k // 128)
        scale_b = active * (ng(cfg.H) * 2 * cfg.I + ng(cfg.I) * cfg.H) * (
            4 + (1 if cfg.wq_zero else 0))
    elif cfg.weight != "fp8":
        scale_b = 0
    elif cfg.fp8_block:                     # one float per 128 x 128 weight block
        nb = lambda n: -(-n // 128)
        scale_b = active * (nb(2 * cfg.I) * nb(cfg.H) + nb(cfg.H) * nb(cfg.I)) * 4
    else:
        scale_b = active * (2 * cfg.I + cfg.H) * 4
    bias_b = active * (2 * cfg.I + cfg.H) * aes if cfg.bias else 0
    x_rows = valid_rows if batched else cfg.M
    x_b = x_rows * cfg.H * aes
    out_rows = valid_rows if batched else cfg.M
    out_b = out_rows * cfg.H * oes
    logit_b = 0 if batched else cfg.M * cfg.E * aes
    z_b = valid_rows * cfg.I * zes
    flops = cfg.flops(valid_rows)
    path_bytes = w13_b + w2_b + scale_b + bias_b + x_b + out_b + logit_b
    # WNA16 dequantises to bf16 and runs bf16 MFMAs
    dt_key = "fp8" if cfg.weight == "fp8" else "bf16" if wq_bits else cfg.weight
    t_hbm = path_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[dt_key] * 1e12)
    t_step = float(np.median(step_ms)) * 1e-3
    t_wall = ms_per_step * 1e-3

    # dominant kernel: W13 GEMM.  Algorithmic bytes: active experts' w13
    # (+ its scales / zero points and bias) and the activation rows it reads
    # once (fp8: the quantised codes and their scales); z is materialised.
    if cfg.weight == "fp8":
        a_scales = (-(-cfg.H // 128) if cfg.fp8_block else 1) * 4
        x_g1 = x_rows * (cfg.H + a_scales)
    else:
        x_g1 = x_b
    w13_extra = 0
    if wq_bits:
        w13_extra = active * -(-cfg.H // 128) * 2 * cfg.I * (4 + (1 if cfg.wq_zero else 0))
    elif cfg.weight == "fp8":
        w13_extra = active * ((2 * cfg.I // 128) * -(-cfg.H // 128) if cfg.fp8_block
                              else 2 * cfg.I) * 4
    if cfg.bias:
        w13_extra += active * 2 * cfg.I * aes
    g1_bytes = w13_b + w13_extra + x_g1
    z_scales = valid_rows * (cfg.I // 128) * 4 if cfg.weight == "fp8" else 0
    materialised = z_b + z_scales
    g1_ms = stage_ms.get("gemm1", float("nan"))
    g1_flops = 2.0 * valid_rows * cfg.H * 2 * cfg.I
    g1_bound = "hbm" if g1_flops / g1_bytes < (MFMA_PEAK_TFLOPS[dt_key] * 1e12) / (
        HBM_PEAK_GBS * 1e9) else "mfma"
    traffic, kname, tsrc, prof_ms = profile_traffic(cfg.name)

    def achieved(ms):
        if g1_bound == "hbm":
            return g1_bytes / (ms * 1e-3) / 1e9
        return g1_flops / (ms * 1e-3) / 1e12
    a = achieved(g1_ms)
    peak = HBM_PEAK_GBS if g1_bound == "hbm" else MFMA_PEAK_TFLOPS[dt_key]
    roof = {"bound": g1_bound, "achieved": round(a, 1), "peak": peak,
            "unit": "GB/s" if g1_bound == "hbm" else "TFLOP/s", "frac": round(a / peak, 4),
            "traffic": traffic,
            "kernel": kname or "GEMM1 (grouped W13 GEMM + SiLU*up)",
            "algorithmic_bytes_per_launch": int(g1_bytes),
            "algorithmic_flops_per_launch": g1_flops,
            "materialised_bytes": int(materialised),
            "avg_launch_ms": round(g1_ms, 4),
            "profile_avg_ms": None if prof_ms is None else round(prof_ms, 4),
            "frac_at_profile_ms": None if prof_ms is None else round(achieved(prof_ms) / peak, 4),
            "traffic_source": tsrc}

    tokens = cfg.M
    value = tokens / (ms_per_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3", "u8": "w8a16_bf16",
                  "u4": "w4a16_bf16"}[cfg.weight],
        "data": "synthetic (seeded; see DESIGN.md input recipe)",
        "config": {"workload": cfg.name, "format": cfg.fmt, "M": cfg.M, "H": cfg.H, "I": cfg.I,
                   "E": cfg.E, "top_k": cfg.top_k, "routing": cfg.scoring,
                   "renormalize": cfg.renormalize, "group_count": cfg.group_count,
                   "k_group": cfg.k_group, "group_select_mode": cfg.group_select_mode,
                   "routed_scaling_factor": cfg.routed_scaling_factor, "bias": cfg.bias,
                   "block_m": info.block_m, "active_experts": active,
                   "valid_rows": valid_rows,
                   **({"local_experts": cfg.local_experts} if cfg.local_experts else {}),
                   **({"fp8_block": cfg.fp8_block} if cfg.fp8_block else {}),
                   **({"weight": cfg.weight, "zero_points": cfg.wq_zero} if wq_bits else {})},
        # whole-path figures on the wall-clock step of the un-instrumented
        # back-to-back forwards (the event-timed steps carry a record between
        # every pair of kernels, which lengthens small steps: decode ~25%)
        "active_tflops": round(flops / t_wall / 1e12, 2),
        "hbm_gbs_path": round(path_bytes / t_wall / 1e9, 1),
        "path_roofline": {"bytes": int(path_bytes), "flops": flops,
                          "t_hbm_us": round(t_hbm * 1e6, 1), "t_mfma_us": round(t_mfma * 1e6, 1),
                          "t_step_us": round(t_wall * 1e6, 1),
                          "t_step_us_median_events": round(t_step * 1e6, 1),
                          "frac": round(max(t_hbm, t_mfma) / t_wall, 4)},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "weight_layout": "packed" if pack_ms is not None else "plain",
        "pack_ms_once": None if pack_ms is None else round(pack_ms, 3),
        "plain_layout_ms_per_step": None if plain_ms is None else round(plain_ms, 4),
        "roofline": roof,
    }

    return res, inp, info


GEMM_SOURCES = ("moe_gemm_common.h", "moe_gemm.hip", "moe_gemm_fp8.hip")


def gemm_source_sha():
    """SHA-256 over the grouped-GEMM sources (in this order), the code the
    committed counter summaries were taken on."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_ffn_router_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size)
    and that kernel's average duration there, or Nones when no summary was
    taken on the current GEMM source."""
    import glob
    import re
    sha = gemm_source_sha()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}.md"))):
        with open(path) as f:
            text = f.read()
        h = re.search(r"^source_sha256: ([0-9a-f]{64})", text, re.M)
        t = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
        k = re.search(r"^dominant_kernel: (.+)$", text, re.M)
        d = re.search(r"^avg_duration_us: ([0-9.]+)", text, re.M)
        if h and t and k and h.group(1) == sha:
            return (int(t.group(1)), k.group(1).strip(), os.path.relpath(path, ROOT),
                    float(d.group(1)) * 1e-3 if d else None)
    return None, None, None, None


def host_cpu():
    """(model name, logical CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(cfg, inp, info, sample):
    import numpy as np
    import oracle
    model, ncpu = host_cpu()
    threads = ncpu                        # every core this process may use
    print(f"[bench] cpu oracle leg on {threads} threads ({model})", file=sys.stderr, flush=True)
    host = {"cpu_model": model, "logical_cpus": ncpu}
    ex = oracle.Experts(inp["w13"].cpu(), inp["w2"].cpu(),
                        None if inp.get("w13_scale") is None else inp["w13_scale"].cpu(),
                        None if inp.get("w2_scale") is None else inp["w2_scale"].cpu(),
                        None if inp.get("w13_bias") is None else inp["w13_bias"].cpu(),
                        None if inp.get("w2_bias") is None else inp["w2_bias"].cpu(),
                        requant_z=cfg.weight == "fp8", block=cfg.fp8_block,
                        bits={"u8": 8, "u4": 4}.get(cfg.weight, 0),
                        w13_zero=None if inp.get("w13_zero") is None else inp["w13_zero"].cpu(),
                        w2_zero=None if inp.get("w2_zero") is None else inp["w2_zero"].cpu())
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    if cfg.fmt == "batched":
        T = inp["max_tokens"]
        counts = inp["expert_num_tokens"].cpu().numpy()
        rows = np.concatenate([e * T + np.arange(c) for e, c in enumerate(counts)])
        n = min(sample or 1536, rows.size)
        rows = rows[:: max(1, rows.size // n)][:n].astype(np.int64)
        t0 = time.perf_counter()
        _, used = oracle.expert_rows(ex, acts, rows, (rows // T).astype(np.int32),
                                     nthreads=threads)
        dt = time.perf_counter() - t0
        # tokens/s equivalent: each token is top_k routed rows
        return {"value": round(n / cfg.top_k / dt, 2), "unit": "tokens/s", "cores": used,
                "kind": "oracle", **host,
                "sample": f"{n} of {int(counts.sum())} valid batched rows (every "
                          f"{max(1, rows.size // n)}th), {dt:.1f}s; tokens = rows / top_k"}
    n = min(sample or 1024, cfg.M)
    logits = inp["logits"].cpu()
    t0 = time.perf_counter()
    ids, w = oracle.route(logits, cfg.top_k, scoring=cfg.scoring, renormalize=cfg.renormalize,
                          group_count=cfg.group_count, k_group=cfg.k_group,
                          group_select_mode=cfg.group_select_mode,
                          routed_scaling_factor=cfg.routed_scaling_factor)
    emap = inp.get("expert_map")
    emap = None if emap is None else emap.cpu().numpy()
    oracle.align(ids, inp["w13"].shape[0], info.block_m, expert_map=emap)
    _, used = oracle.forward_tokens(ex, acts, ids, w, tokens=np.arange(n), nthreads=threads,
                                    expert_map=emap)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
            **host,
            "sample": f"routing + align of all {cfg.M} tokens, expert FFN of the first {n} "
                      f"tokens, {dt:.1f}s"}


if __name__ == "__main__":
    main()
