"""Seeded random sweep at larger shapes than test_gpu_sweep.py: M 100-3000
tokens, H 512-2048, I 256-1408, E 8-256 experts, top_k up to 8, contiguous
and batched (uniform or Zipf-skewed slabs), bf16, fp8 per channel and
block-wise, 8- and 4-bit WNA16 (groups of 32 / 64 / 128, with and without
zero points), the library's own tile choice.  Routing and align are checked
bit for bit over every token; outputs on a sample (42 tokens, or 202 slab
rows) against the oracle within the dtype's bound."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 80


def draw(i: int) -> W.MoeConfig:
    rng = np.random.default_rng(9100 + i)
    pick = lambda seq: seq[int(rng.integers(len(seq)))]
    weight = pick(["bf16", "bf16", "fp8", "fp8_block", "u8", "u4"])
    fmt = "batched" if rng.random() < 0.35 else "contiguous"
    E = pick([8, 16, 64, 128, 256])
    top_k = int(rng.integers(1, min(8, E) + 1))
    H = pick([512, 1024, 2048])
    I = pick([256, 512, 768, 1024, 1408])
    M = int(rng.integers(100, 3000))
    kw = dict(name=f"large{i}_{fmt}_{weight}", M=M, H=H, I=I, E=E, top_k=top_k, fmt=fmt,
              bias=bool(rng.random() < 0.3))
    if weight == "fp8_block":
        kw.update(weight="fp8", fp8_block=128)
    else:
        kw.update(weight=weight)
    if weight in ("u8", "u4"):
        kw.update(wq_zero=bool(rng.random() < 0.5), wq_group=pick([32, 64, 128]))
    kw.update(scoring=pick(["softmax", "sigmoid"]), renormalize=bool(rng.random() < 0.5))
    if fmt == "batched":
        kw.update(zipf_s=pick([0.0, 1.1]))
    return W.MoeConfig(**kw)


@pytest.mark.parametrize("i", range(N_CASES))
def test_large_random_combination(i):
    cfg = draw(i)
    dev = GH.device()
    print(f"[case] large sweep {i}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, 9200 + i, device=dev)
    packed = cfg.weight in ("bf16", "fp8")
    rng = np.random.default_rng(i)
    if cfg.fmt == "contiguous":
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=packed)
        ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        tokens = np.unique(np.concatenate([[0, cfg.M - 1], rng.choice(cfg.M, 40, replace=False)]))
        GH.check_output(inp, out, ids_o, w_o, tokens=tokens, what=f"large sweep {i}")
        return
    out, ws, info = GH.run_batched(inp, dev, reduce=False, out_dtype=torch.float32,
                                   packed=packed)
    GH.check_batched_tilelist(inp, ws, info)
    rows, experts = GH.batched_rows(inp)
    sel = np.unique(np.concatenate([[0, len(rows) - 1],
                                    rng.choice(len(rows), min(200, len(rows)), replace=False)]))
    rows, experts = rows[sel], experts[sel]
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    ref, ties = GH.ref_rows(inp, acts, rows, experts)
    got = out.float().reshape(-1, cfg.H)[torch.as_tensor(rows, device=dev)].cpu().numpy()
    GH.compare(cfg, got, ref, what=f"large sweep {i} slab rows", ties=ties)
