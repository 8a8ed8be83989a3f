"""Parity at the full workload sizes, in the launch configuration the
benchmark times.  Every routing / align result is compared bit for bit.
Outputs are checked tile by tile: for every (expert, row chunk) tile of
every chunk height the GEMM families use, the expert output of the chunk's
first and last routed rows (all columns) against the oracle's expert FFN;
then the final output of a token sample (first, last, and tokens of those
items) against the oracle's weighted sum."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

FULL = [W.TINY_F32, W.MIXTRAL_PREFILL, W.DECODE_SMALL_EXPERTS, W.DEEPSEEK_GROUPED]


def _token_sample(M, item_tokens, n=32, seed=0):
    """First and last token plus up to n tokens that own sampled tile rows."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(item_tokens, size=min(n, item_tokens.size), replace=False)
    return np.unique(np.concatenate([[0, M - 1], pick])).astype(np.int64)


def _margin(inp):
    """The k_group-boundary near-tie report on the logits this run used."""
    cfg = inp["cfg"]
    if cfg.group_count > 1 and cfg.group_select_mode == 1:
        from test_routing_margin import margin_report
        margin_report(inp["logits"].cpu(), cfg)


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_full_size_contiguous(cfg):
    dev = GH.device()
    seed = 1000 + W.CONFIGS.index(cfg)
    print(f"[case] {cfg.name} seed={seed} generating", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    print(f"[case] {cfg.name} ran; block_m={info.block_m}", flush=True)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    assert GH.B.device_status(ws, info) == 0
    _margin(inp)
    counts = np.bincount(ids_o.ravel(), minlength=cfg.E)
    print(f"[case] {cfg.name} active experts={int((counts > 0).sum())} "
          f"rows/expert max={counts.max()} min={counts.min()}", flush=True)
    if cfg.M <= 64:
        GH.check_z_all_contiguous(inp, ws, info, ids_o, dev, "full, every item's z")
        GH.check_output(inp, out, ids_o, w_o, what="full")
    else:
        item_tokens = GH.check_tiles_contiguous(inp, ws, info, dev)
        GH.check_output(inp, out, ids_o, w_o, tokens=_token_sample(cfg.M, item_tokens),
                        what="full")
    if cfg.out_dtype == "bf16":
        out16, _, _ = GH.run_contiguous(inp, dev)
        GH.check_rounded(out16, out)


@pytest.mark.parametrize("packed", [False, True], ids=["plain", "packed"])
def test_full_size_batched_fp8(packed):
    cfg = W.BATCHED_FP8
    dev = GH.device()
    seed = 1000 + W.CONFIGS.index(cfg)
    print(f"[case] {cfg.name} seed={seed} packed={packed} generating", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    counts = inp["expert_num_tokens"].cpu().numpy()
    print(f"[case] {cfg.name} rows/expert max={counts.max()} min={counts.min()} "
          f"total={counts.sum()}", flush=True)
    out, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32, packed=packed)
    GH.check_batched_tilelist(inp, ws, info)
    assert GH.B.device_status(ws, info) == 0
    rows = GH.check_tiles_batched(inp, ws, info, out, dev)
    out16, _, _ = GH.run_batched(inp, dev, packed=packed)
    idx = torch.as_tensor(rows, device=dev)
    GH.check_rounded(out16.reshape(-1, cfg.H)[idx], out.reshape(-1, cfg.H)[idx])
    # invalid (NaN-filled) rows never leak into valid outputs
    valid = torch.as_tensor(GH.batched_rows(inp)[0], device=dev)
    assert torch.isfinite(out.reshape(-1, cfg.H)[valid]).all()


def test_full_size_ep8_shard():
    """One rank of the DeepSeek-like layer under 8-way expert parallelism
    (32768 tokens routed over 256 experts, 32 held here), in the launch
    configuration the benchmark times: global ids and local align bit for
    bit, every tile's rows and sampled output rows against the oracle's
    partial sums."""
    cfg = W.EP8_SHARD
    dev = GH.device()
    seed = 1100 + W.EXTRA.index(cfg)
    print(f"[case] {cfg.name} seed={seed} generating", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    emap = inp["expert_map"]
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, expert_map=emap)
    ids_o, w_o = GH.oracle_route(inp)
    M, K, E = cfg.M, cfg.top_k, cfg.local_experts
    ids_g = GH.region(ws, info.off_topk_ids, torch.int32, M * K).reshape(M, K)
    assert np.array_equal(ids_g, ids_o)
    emap_np = emap.cpu().numpy()
    counts_o, sorted_o, eids_o, npp_o = oracle.align(ids_o, E, info.block_m, expert_map=emap_np)
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    assert npp == npp_o
    assert np.array_equal(GH.region(ws, info.off_expert_counts, torch.int32, E), counts_o)
    assert np.array_equal(GH.region(ws, info.off_sorted_ids, torch.int32, npp), sorted_o)
    assert GH.B.device_status(ws, info) == 0
    _margin(inp)
    print(f"[case] {cfg.name} local rows={int(counts_o.sum())} max/expert={counts_o.max()}",
          flush=True)
    item_tokens = GH.check_tiles_contiguous(inp, ws, info, dev, E_local=E)
    tokens = _token_sample(M, item_tokens)
    acts = oracle.Acts(inp["hidden"].cpu())
    y, _ = oracle.forward_tokens(GH.oracle_experts(inp), acts, ids_o, w_o, tokens=tokens,
                                 expert_map=emap_np)
    GH.compare(cfg, out.cpu().numpy()[tokens], y, what="ep8 shard")


def test_full_size_mixtral_m4096():
    """The Mixtral-shaped layer at M 4096 (about 1024 rows per expert: the
    256-row tiles), every tile's rows and a token sample."""
    cfg = W.MIXTRAL_M4096
    dev = GH.device()
    seed = 1100 + W.EXTRA.index(cfg)
    print(f"[case] {cfg.name} seed={seed} generating", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    assert GH.B.device_status(ws, info) == 0
    item_tokens = GH.check_tiles_contiguous(inp, ws, info, dev)
    GH.check_output(inp, out, ids_o, w_o, tokens=_token_sample(cfg.M, item_tokens),
                    what="full mixtral m4096")
    out16, _, _ = GH.run_contiguous(inp, dev)
    GH.check_rounded(out16, out)


def test_full_size_block_fp8():
    """The DeepSeek-like layer with block-wise fp8 weights (128 x 128 blocks)
    and in-path per (token, 128 columns) activation quantisation."""
    cfg = W.DEEPSEEK_BLOCKFP8
    dev = GH.device()
    seed = 1100 + W.EXTRA.index(cfg)
    print(f"[case] {cfg.name} seed={seed} generating", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    print(f"[case] {cfg.name} ran", flush=True)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    item_tokens = GH.check_tiles_contiguous(inp, ws, info, dev)
    GH.check_output(inp, out, ids_o, w_o, tokens=_token_sample(cfg.M, item_tokens),
                    what="full block fp8")
    out16, _, _ = GH.run_contiguous(inp, dev)
    GH.check_rounded(out16, out)
