"""Parity of the contiguous-format variants the pages name beside the plain
forward: an expert-parallel shard (expert map, FlagGems walkthrough's
expert_id == -1 and the vLLM page's expert map), the routing weight applied
to the first layer's output (apply_router_weight_on_input, walkthrough
sec. 1.2) and chunked execution (the walkthrough's CHUNK_SIZE).  Ids, counts
and sorted ids bit for bit, outputs within the dtype tolerance of the
oracle run with the same options."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu


def _shard(inp, own):
    """The workload restricted to the experts `own` (local slot i = own[i])."""
    loc = dict(inp)
    for name in ("w13", "w2", "w13_bias", "w2_bias", "w13_scale", "w2_scale"):
        if inp.get(name) is not None:
            loc[name] = inp[name][torch.as_tensor(own)].contiguous()
    return loc


def _emap(Eg, own):
    m = np.full(Eg, -1, np.int32)
    m[np.asarray(own)] = np.arange(len(own), dtype=np.int32)
    return m


SHARD_CASES = [
    # name, cfg, own experts (global ids, in local-slot order), packed
    ("bf16_shard", W.DECODE_SMALL_EXPERTS.scaled(name="ep_bf16", M=96, H=256, I=256, E=32,
                                                 top_k=4), [5, 3, 17, 30, 9, 0, 22, 11], False),
    ("bf16_shard_prefill_tiles", W.MIXTRAL_PREFILL.scaled(name="ep_prefill", M=400, H=128, I=256,
                                                          E=16, top_k=2),
     list(range(8, 16)), True),
    ("grouped_sigmoid_shard", W.DEEPSEEK_GROUPED.scaled(name="ep_grouped", M=64, H=256, I=128,
                                                        E=64), list(range(16, 32)), False),
    ("fp8_shard", W.MIXTRAL_PREFILL.scaled(name="ep_fp8", M=200, H=256, I=256, E=16, top_k=2,
                                           weight="fp8"), [1, 4, 6, 15], True),
]


@pytest.mark.parametrize("case", SHARD_CASES, ids=[c[0] for c in SHARD_CASES])
def test_expert_shard_parity(case):
    name, cfg, own, packed = case
    dev = GH.device()
    print(f"[case] shard {name} own={own} packed={packed}", flush=True)
    inp = W.make_inputs(cfg, 3000 + SHARD_CASES.index(case))
    emap = _emap(cfg.E, own)
    loc = _shard(inp, own)
    out, ws, info = GH.run_contiguous(loc, dev, out_dtype=torch.float32, packed=packed,
                                      expert_map=torch.as_tensor(emap).to(dev))
    # global routing, bit for bit
    ids_o, w_o = GH.oracle_route(inp)
    M, K = cfg.M, cfg.top_k
    ids_g = GH.region(ws, info.off_topk_ids, torch.int32, M * K).reshape(M, K)
    assert np.array_equal(ids_g, ids_o)
    # local align, bit for bit
    E = len(own)
    counts_o, sorted_o, eids_o, npp_o = oracle.align(ids_o, E, info.block_m, expert_map=emap)
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    assert npp == npp_o
    assert np.array_equal(GH.region(ws, info.off_expert_counts, torch.int32, E), counts_o)
    assert np.array_equal(GH.region(ws, info.off_sorted_ids, torch.int32, npp), sorted_o)
    assert np.array_equal(GH.region(ws, info.off_expert_ids, torch.int32, npp // info.block_m),
                          eids_o)
    # this shard's partial sums
    y, ties = GH.ref_tokens(loc, ids_o, w_o, expert_map=emap)
    GH.compare(cfg, out.float().cpu().numpy(), y, what=name, ties=ties)


def test_expert_shards_sum_to_the_full_layer():
    """Four shards of 8 of 32 experts: their partial outputs add up to the
    unsharded forward (same routing), within the bf16 bar."""
    dev = GH.device()
    cfg = W.DECODE_SMALL_EXPERTS.scaled(name="ep_sum", M=64, H=256, I=256, E=32, top_k=4)
    inp = W.make_inputs(cfg, 3100)
    full, _, _ = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    total = torch.zeros_like(full)
    rng = np.random.default_rng(3)
    perm = rng.permutation(cfg.E)
    for rank in range(4):
        own = perm[rank * 8:(rank + 1) * 8].tolist()
        part, _, _ = GH.run_contiguous(_shard(inp, own), dev, out_dtype=torch.float32,
                                       expert_map=torch.as_tensor(_emap(cfg.E, own)).to(dev))
        total += part
    ids_o, w_o = GH.oracle_route(inp)
    acts = oracle.Acts(inp["hidden"].cpu())
    y, _ = oracle.forward_tokens(GH.oracle_experts(inp), acts, ids_o, w_o)
    GH.compare(cfg, total.cpu().numpy(), y, what="sum of shards")
    GH.compare(cfg, full.cpu().numpy(), y, what="unsharded")


WOI_CASES = [
    W.MIXTRAL_PREFILL.scaled(name="woi_bf16_bias", M=96, H=256, I=512, bias=True),
    W.MIXTRAL_PREFILL.scaled(name="woi_bf16_prefill_tiles", M=384, H=128, I=256, E=4),
    W.DECODE_SMALL_EXPERTS.scaled(name="woi_decode", M=8, H=256, I=128, E=32, top_k=4, bias=True),
    W.MIXTRAL_PREFILL.scaled(name="woi_fp8_bias", M=64, H=256, I=256, weight="fp8", bias=True),
    W.TINY_F32.scaled(name="woi_f32", bias=True),
]


@pytest.mark.parametrize("cfg", WOI_CASES, ids=[c.name for c in WOI_CASES])
@pytest.mark.parametrize("packed", [False, True])
def test_weight_on_input_parity(cfg, packed):
    if packed and cfg.weight == "f32":
        pytest.skip("packing is for bf16 / fp8 weights")
    dev = GH.device()
    print(f"[case] weight on input {cfg.name} packed={packed}", flush=True)
    inp = W.make_inputs(cfg, 3200 + WOI_CASES.index(cfg))
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=packed,
                                      apply_weight_on_input=True)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    y, ties = GH.ref_tokens(inp, ids_o, w_o, weight_on_input=True)
    GH.compare(cfg, out.float().cpu().numpy(), y, what="weight on input", ties=ties)


@pytest.mark.parametrize("routing", ["router", "precomputed", "inplace"])
def test_chunked_equals_unchunked(routing):
    """Chunks of 64 tokens (the last one ragged) give the unchunked output
    bit for bit: every output row is computed from its own token alone, in
    the same order."""
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name="chunked", M=300, H=256, I=512, E=8, bias=True)
    inp = W.make_inputs(cfg, 3300)
    pre = None
    if routing != "router":
        rng = np.random.default_rng(9)
        ids = np.stack([rng.permutation(cfg.E)[:cfg.top_k] for _ in range(cfg.M)]).astype(np.int32)
        pre = (ids, rng.random((cfg.M, cfg.top_k)).astype(np.float32))
    print(f"[case] chunked {routing}", flush=True)
    full, _, _ = GH.run_contiguous(inp, dev, precomputed=pre)
    chunked, _, info = GH.run_contiguous(inp, dev, precomputed=pre, chunk_tokens=64,
                                         inplace=routing == "inplace")
    assert info.max_sorted_len == 64 * cfg.top_k + cfg.E * 15
    assert torch.equal(full, chunked)
