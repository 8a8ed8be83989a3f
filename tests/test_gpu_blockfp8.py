"""Block-wise fp8 W8A8 (one scale per 128 x 128 weight block, activations
quantised per token and 128 columns in the path) against the CPU oracle.

Outputs within 6e-2 x RMS of the oracle's double result; the in-path
activation codes and group scales bit for bit; routing and align bit for bit
as everywhere else."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

BLOCK_SMALL = [
    # H 320: a short last K block (64 columns); several z column blocks
    W.MIXTRAL_PREFILL.scaled(name="blk_short_k", M=64, H=320, I=256, weight="fp8",
                             fp8_block=128),
    # 256 rows per expert: two row chunks per expert; biases
    W.MIXTRAL_PREFILL.scaled(name="blk_chunks_bias", M=512, H=256, I=384, E=4, weight="fp8",
                             fp8_block=128, bias=True),
    # grouped sigmoid routing with skewed experts, as the DeepSeek-like layer
    W.DEEPSEEK_GROUPED.scaled(name="blk_grouped", M=96, H=512, I=256, E=32, weight="fp8",
                              fp8_block=128),
]


@pytest.mark.parametrize("cfg", BLOCK_SMALL, ids=[c.name for c in BLOCK_SMALL])
@pytest.mark.parametrize("seed_off", [0, 1000])
def test_block_fp8_small_parity(cfg, seed_off):
    dev = GH.device()
    seed = 3000 + BLOCK_SMALL.index(cfg) + seed_off
    print(f"[case] {cfg.name} seed={seed}", flush=True)
    inp = W.make_inputs(cfg, seed)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, out, ids_o, w_o, what=f"seed{seed}")
    out16, _, _ = GH.run_contiguous(inp, dev)
    GH.check_rounded(out16, out)


def test_block_fp8_activation_codes_bit_exact():
    """In-path block quantisation: per (token, 128 columns) scale amax / 448,
    RNE, saturating; an all-zero group gets scale 1; a short last group."""
    import oracle
    dev = GH.device()
    cfg = BLOCK_SMALL[0].scaled(name="blk_codes", M=80)
    inp = W.make_inputs(cfg, 3100)
    inp["hidden"][5, 128:256] = 0.0
    inp["hidden"][7, :128] *= 300.0
    _, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    q_ref, s_ref = oracle.quant_rows_fp8(inp["hidden"].float().numpy(), block=128)
    ng = -(-cfg.H // 128)
    q = GH.region(ws, info.off_aq, torch.uint8, cfg.M * cfg.H).reshape(cfg.M, cfg.H)
    s = GH.region(ws, info.off_aq_scale, torch.float32, cfg.M * ng).reshape(cfg.M, ng)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


BATCHED_BLOCK = W.BATCHED_FP8.scaled(name="batched_blk_small", M=96, H=384, I=256, E=8, top_k=2,
                                     fp8_block=128)


@pytest.mark.parametrize("reduce", [False, True])
def test_block_fp8_batched_bf16_activations(reduce):
    """Batched slabs of bf16 activations, quantised in the path at their
    padded positions with group scales."""
    import oracle
    dev = GH.device()
    inp = W.make_inputs(BATCHED_BLOCK, 3200)
    out, ws, info = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32)
    GH.check_batched_tilelist(inp, ws, info)
    ex = GH.oracle_experts(inp)
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=True, block=128)
    if reduce:
        y, _, ties = oracle.forward_tokens(ex, oracle.Acts(inp["tokens"].cpu(), quantize=True,
                                                           block=128),
                                           inp["topk_ids"].cpu().numpy(),
                                           inp["token_map_w"].cpu().double().numpy(),
                                           tie_window=GH.TIE_WINDOW)
        GH.compare(BATCHED_BLOCK, out.cpu().numpy(), y, "batched block reduce", ties=ties)
    else:
        rows, experts = GH.batched_rows(inp)
        ref, _, ties = oracle.expert_rows(ex, acts, rows, experts, tie_window=GH.TIE_WINDOW)
        got = out.reshape(-1, BATCHED_BLOCK.H)[torch.as_tensor(rows, device=out.device)]
        GH.compare(BATCHED_BLOCK, got.cpu().numpy(), ref, "batched block rows", ties=ties)


def test_block_fp8_batched_prequantised_activations():
    """Batched slabs of fp8 codes with caller-side group scales
    [E, max_tokens, ceil(H / 128)] (quantised here with a torch cast)."""
    import oracle
    from mixture_experts_ffn_router_amd import binding as B
    dev = GH.device()
    cfg = BATCHED_BLOCK
    inp = W.make_inputs(cfg, 3300)
    E, T, H = inp["hidden"].shape
    ng = -(-H // 128)
    x = inp["hidden"].float().nan_to_num(0.0)
    xp = torch.nn.functional.pad(x, (0, ng * 128 - H)).view(E, T, ng, 128)
    amax = xp.abs().amax(-1)
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (xp / sc[..., None]).view(E, T, ng * 128)[..., :H].to(torch.float8_e4m3fn)
    pw = B.pack_weights(inp["w13"].to(dev), inp["w2"].to(dev))
    out, ws, info = B.fused_moe_batched(codes.to(dev), inp["expert_num_tokens"].to(dev), pw, None,
                                        M=cfg.M, top_k=cfg.top_k, a_scale=sc.to(dev).contiguous(),
                                        w13_scale=inp["w13_scale"].to(dev),
                                        w2_scale=inp["w2_scale"].to(dev),
                                        out_dtype=torch.float32, fp8_block=128)
    torch.cuda.synchronize()
    rows, experts = GH.batched_rows(inp)
    ex = GH.oracle_experts(inp)
    acts = oracle.Acts(codes.cpu(), scale=sc.cpu(), block=128)
    ref, _, ties = oracle.expert_rows(ex, acts, rows, experts, tie_window=GH.TIE_WINDOW)
    got = out.reshape(-1, H)[torch.as_tensor(rows, device=out.device)]
    GH.compare(cfg, got.cpu().numpy(), ref, "batched block prequantised", ties=ties)
