"""The intermediate z (SiLU(gate) * up, the first GEMM's output) read back
from the workspace and compared with the oracle's, for every routed item of
small cases: float32 and bf16 z value by value, and on the fp8 path, where
z is quantised again before the second GEMM (FlagGems walkthrough, "FP8
W8A8"; here per row and 128 columns), its codes and group scales.  The bars
(gpu_harness: Z_REL, Z_RMS and the check_z_codes constants) and why they are
what they are sit with the harness; the full-size tile checks apply the same
comparison to every (expert, row chunk) tile's first and last rows."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

CONTIG = [
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_fp8", M=96, H=256, I=384, E=8, top_k=2,
                              weight="fp8", bias=True), False),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_fp8_packed", M=300, H=208, I=256, E=4, top_k=2,
                              weight="fp8", bias=True), True),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_blockfp8", M=80, H=384, I=256, E=8, top_k=2,
                              weight="fp8", fp8_block=128), True),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_bf16", M=200, H=256, I=320, E=8, top_k=2,
                              bias=True), False),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_bf16_packed", M=300, H=256, I=256, E=4, top_k=2),
     True),
    (W.TINY_F32.scaled(name="z_contig_f32", bias=True), False),
]


@pytest.mark.parametrize("case", CONTIG, ids=[c[0].name for c in CONTIG])
def test_z_contiguous(case):
    cfg, packed = case
    dev = GH.device()
    print(f"[case] z {cfg.name} packed={packed}", flush=True)
    inp = W.make_inputs(cfg, 4100 + CONTIG.index(case))
    _, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=packed)
    ids_o, _ = GH.check_routing_and_align(inp, ws, info)
    GH.check_z_all_contiguous(inp, ws, info, ids_o, dev, cfg.name)


@pytest.mark.parametrize("weight", ["fp8", "bf16"])
def test_z_batched_skewed(weight):
    """Batched slabs, one expert past two 128-row tiles, packed weights."""
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name=f"z_batched_{weight}", M=400, H=256, I=384, E=4, top_k=2,
                               weight=weight)
    inp = W.make_inputs(cfg, 4200)
    counts = inp["expert_num_tokens"].cpu().numpy()
    print(f"[case] z batched {weight} counts={counts.tolist()}", flush=True)
    assert counts.max() > 256
    _, ws, info = GH.run_batched(inp, dev, reduce=False, out_dtype=torch.float32, packed=True)
    GH.check_batched_tilelist(inp, ws, info)
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    sorted_ids = GH.region(ws, info.off_sorted_ids, torch.int32, npp)
    T = inp["max_tokens"]
    pos = np.nonzero(sorted_ids < cfg.E * T)[0]
    rows = sorted_ids[pos].astype(np.int64)
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=weight == "fp8")
    GH.check_z(inp, ws, info, acts, rows, (rows // T).astype(np.int32), pos, dev, cfg.name)
