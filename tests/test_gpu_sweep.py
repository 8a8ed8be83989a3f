"""Seeded random sweep over the combination matrix of the fused MoE forward:
input format x weight type (f32, bf16, fp8 per channel or per 128 x 128
block, 8- and 4-bit WNA16 codes with or without zero points and groups of
32 / 64 / 128 K rows) x routing (softmax / sigmoid, renormalised or not,
grouped selection in either mode, routed_scaling_factor) x biases x top_k x
ragged sizes x tile family x packed / plain weights x chunked execution x
routing weight on the input.  Every case is checked against the CPU oracle:
routing and align bit for bit, the output within its dtype's tolerance.
The vLLM modular-kernel page describes the same strategy (every compatible
combination of implementation choices checked against a reference)."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 160


def draw(i: int) -> tuple:
    """Case i: (config, run options).  Only combinations the boundary accepts."""
    rng = np.random.default_rng(7100 + i)
    pick = lambda seq: seq[int(rng.integers(len(seq)))]
    weight = pick(["bf16", "bf16", "fp8", "fp8_block", "u8", "u4", "f32"])
    fmt = "contiguous" if weight == "f32" or rng.random() < 0.6 else "batched"
    E = pick([4, 8, 16, 32, 64])
    top_k = int(rng.integers(1, min(8, E) + 1))
    H = pick([64, 128, 208, 256, 384])
    I = pick([128, 256, 384]) if weight.startswith("fp8") else pick([64, 96, 128, 192, 256])
    M = int(rng.integers(1, 260))
    kw = dict(name=f"sweep{i}_{fmt}_{weight}", M=M, H=H, I=I, E=E, top_k=top_k, fmt=fmt,
              bias=bool(rng.random() < 0.4))
    if weight == "f32":
        kw.update(act="f32", weight="f32")
    elif weight == "fp8_block":
        kw.update(weight="fp8", fp8_block=128)
    else:
        kw.update(weight=weight)
    if weight in ("u8", "u4"):
        kw.update(wq_zero=bool(rng.random() < 0.5), wq_group=pick([32, 64, 128]))
    kw.update(scoring=pick(["softmax", "sigmoid"]), renormalize=bool(rng.random() < 0.5),
              routed_scaling_factor=pick([1.0, 2.5]))
    if fmt == "contiguous" and rng.random() < 0.4:
        groups = [G for G in (2, 4, 8) if E % G == 0 and E // G >= 2 and G <= E]
        if groups:
            G = pick(groups)
            kg = int(rng.integers(1, G + 1))
            if top_k <= kg * (E // G):
                kw.update(group_count=G, k_group=kg, group_select_mode=int(rng.integers(0, 2)),
                          expert_bias_var=0.5)
    if fmt == "batched":
        kw.update(zipf_s=pick([0.0, 1.1]))
    opts = {}
    if weight == "bf16":
        opts["packed"] = bool(rng.random() < 0.5)
        if rng.random() < 0.5:
            # (the GEMM1 width hint is a contiguous-format argument of the binding)
            tiles = ["dma160", "reg64", "reg16", "dma32", "dma64", "dma256"]
            opts["tile"] = pick(tiles + (["dma160/wc2"] if fmt == "contiguous" else []))
    elif weight in ("u8", "u4") and rng.random() < 0.5:
        opts["tile"] = pick(["dma32", "dma64", "dma160"])
    elif weight == "fp8":
        opts["packed"] = bool(rng.random() < 0.5)
    if fmt == "contiguous":
        if M > 8 and rng.random() < 0.3:
            opts["chunk_tokens"] = int(rng.integers(1, M))
        if rng.random() < 0.2:
            opts["apply_weight_on_input"] = True
    else:
        opts["reduce"] = bool(rng.random() < 0.5)
    return W.MoeConfig(**kw), opts


def _run_options(opts):
    extra = {}
    if "tile" in opts:
        extra.update(GH.tile_kwargs(opts["tile"]))
    return extra


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_combination(i):
    cfg, opts = draw(i)
    dev = GH.device()
    print(f"[case] sweep {i}: {cfg} {opts}", flush=True)
    inp = W.make_inputs(cfg, 7200 + i)
    extra = _run_options(opts)
    out_dtype = torch.float32
    if cfg.fmt == "contiguous":
        woi = opts.get("apply_weight_on_input", False)
        for k in ("chunk_tokens", "apply_weight_on_input"):
            if k in opts:
                extra[k] = opts[k]
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=out_dtype,
                                          packed=opts.get("packed", False), **extra)
        if opts.get("chunk_tokens"):
            ids_o, w_o = GH.oracle_route(inp)        # the workspace holds the last chunk only
        else:
            ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        y, ties = GH.ref_tokens(inp, ids_o, w_o, weight_on_input=woi)
        GH.compare(cfg, out.float().cpu().numpy(), y, what=f"sweep {i}", ties=ties)
        return
    reduce = opts["reduce"]
    out, ws, info = GH.run_batched(inp, dev, reduce=reduce, out_dtype=out_dtype,
                                   packed=opts.get("packed", False), **extra)
    GH.check_batched_tilelist(inp, ws, info)
    rows, experts = GH.batched_rows(inp)
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    o_ref, ties = GH.ref_rows(inp, acts, rows, experts)
    if not reduce:
        got = out.float().cpu().numpy().reshape(-1, cfg.H)[rows]
        GH.compare(cfg, got, o_ref, what=f"sweep {i} slab rows", ties=ties)
        return
    y, yties = GH.reduce_rows(inp, rows, o_ref, ties)
    GH.compare(cfg, out.float().cpu().numpy(), y, what=f"sweep {i} reduce", ties=yties)
