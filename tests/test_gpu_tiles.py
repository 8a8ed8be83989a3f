"""Tile-schedule coverage at small sizes, every output compared.

The persistent GEMMs walk their tiles in groups of 8 row chunks per expert,
pipeline the next tile's first K stages behind a finished tile, and switch
the weight cache policy per tile (an expert with one row chunk is the only
reader of its weights).  These cases make all of that happen with outputs
the oracle computes in seconds:
  * one expert of 1300 rows (9 chunks of 160 rows, 11 of 128): the walk's
    full-group branch plus a remainder group;
  * experts of 100, 400 and 1000 rows beside it: single- and multi-chunk
    tiles (both cache policies) in one launch;
  * enough column tiles (wide I for the first GEMM, wide H for the second)
    that the tiles outnumber the workgroups several times, so every
    workgroup runs many tiles back to back.
Each shape runs the oracle once and checks every variant against it."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

M_SKEW = 1400


def skewed_routing(M=M_SKEW, seed=5):
    """Precomputed top-2 ids over 4 experts: expert 0 gets tokens [0, 1300),
    expert 1 [0, 100), expert 2 [100, 400) and [1300, 1400), expert 3
    [400, 1400); weights uniform in (0, 1)."""
    t = np.arange(M)
    ids = np.empty((M, 2), np.int32)
    ids[:, 0] = np.where(t < 1300, 0, 2)
    ids[:, 1] = np.select([t < 100, t < 400, t < 1300], [1, 2, 3], 3)
    w = np.random.default_rng(seed).uniform(0.05, 1.0, (M, 2)).astype(np.float32)
    return ids, w


_REF = {}


def _oracle_y(inp, ids, w, key):
    """(oracle output, its fp8 near-tie report or None), cached by key."""
    if key not in _REF:
        _REF[key] = GH.ref_tokens(inp, ids, w.astype(np.float64))
    return _REF[key]


BF16_SHAPES = {"gemm1_wide": dict(H=256, I=2560), "gemm2_wide": dict(H=6144, I=256)}


@pytest.mark.parametrize("shape", list(BF16_SHAPES))
def test_bf16_many_chunks_many_tiles(shape):
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name=f"tiles_bf16_{shape}", M=M_SKEW, E=4, bias=True,
                                   **BF16_SHAPES[shape])
    inp = W.make_inputs(cfg, 91)
    ids, w = skewed_routing()
    y, ties = _oracle_y(inp, ids, w, cfg.name)
    outs = {}
    for tile in ("auto", "dma160/wc2", "dma160/wc4", "dma256"):
        for packed in (False, True):
            print(f"[case] {cfg.name} tile={tile} packed={packed}", flush=True)
            out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w),
                                              out_dtype=torch.float32, packed=packed,
                                              **GH.tile_kwargs(tile))
            GH.check_routing_and_align(inp, ws, info, ids_o=ids, w_o=w.astype(np.float64))
            GH.compare(cfg, out.cpu().numpy(), y, f"{tile} packed={packed}", ties=ties)
            outs[(tile, packed)] = out
        assert torch.equal(outs[(tile, False)], outs[(tile, True)]), tile


def test_fp8_contiguous_many_chunks_many_tiles():
    """fp8 per-channel and block-wise (128 x 128) weights on the packed fp8
    kernels (128-row tiles, 256 columns): GEMM1 with 32 column tiles per
    chunk, then GEMM2 with 24.  The comparison takes the z codes that lie on
    a rounding tie either way (the oracle's near-tie report): one such flip
    moves an output by about (1/8)(|z| / RMS z)(4 / sqrt(I)) of the RMS."""
    dev = GH.device()
    ids, w = skewed_routing()
    for shape, dims in (("gemm1_wide", dict(H=256, I=4096)),
                        ("gemm2_wide", dict(H=6144, I=2048))):
        for blk in (0, 128):
            cfg = W.MIXTRAL_PREFILL.scaled(name=f"tiles_fp8_{shape}_b{blk}", M=M_SKEW, E=4,
                                           weight="fp8", fp8_block=blk, bias=True, **dims)
            inp = W.make_inputs(cfg, 92)
            y, ties = _oracle_y(inp, ids, w, cfg.name)
            print(f"[case] {cfg.name}", flush=True)
            out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w),
                                              out_dtype=torch.float32, packed=True)
            GH.check_routing_and_align(inp, ws, info, ids_o=ids, w_o=w.astype(np.float64))
            GH.compare(cfg, out.cpu().numpy(), y, "every token", ties=ties)


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_batched_many_chunks_many_tiles(packed):
    """Batched fp8 slabs with the same skewed rows (1300 / 100 / 400 / 1000)
    and NaN past each count, every valid row compared."""
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="tiles_fp8_batched", M=M_SKEW, E=4, top_k=2, H=256,
                               I=4096, max_tokens=1408)
    gen = torch.Generator().manual_seed(93)
    counts = torch.tensor([1300, 100, 400, 1000], dtype=torch.int32)
    T = cfg.max_tokens
    xb = torch.full((cfg.E, T, cfg.H), float("nan"))
    for e, c in enumerate(counts.tolist()):
        xb[e, :c] = torch.randn(c, cfg.H, generator=gen)
    w13 = torch.randn(cfg.E, cfg.H, 2 * cfg.I, generator=gen) / cfg.H ** 0.5
    w2 = torch.randn(cfg.E, cfg.I, cfg.H, generator=gen) / cfg.I ** 0.5
    q13, s13 = W.quantize_weight_fp8(w13)
    q2, s2 = W.quantize_weight_fp8(w2)
    inp = {"cfg": cfg, "hidden": xb.to(torch.bfloat16), "expert_num_tokens": counts,
           "w13": q13, "w2": q2, "w13_scale": s13, "w2_scale": s2, "max_tokens": T,
           "w13_bias": None, "w2_bias": None}
    print(f"[case] {cfg.name} packed={packed}", flush=True)
    out, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32, packed=packed)
    GH.check_batched_tilelist(inp, ws, info)
    rows, experts = GH.batched_rows(inp)
    acts = oracle.Acts(inp["hidden"], quantize=True)
    ref, ties = GH.ref_rows(inp, acts, rows, experts)
    got = out.reshape(-1, cfg.H)[torch.as_tensor(rows, device=dev)].cpu().numpy()
    GH.compare(cfg, got, ref, "every valid slab row", ties=ties)
    assert B.device_status(ws, info) == 0
