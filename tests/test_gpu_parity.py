"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: topk ids, per-expert counts, sorted ids, expert ids and
num_post_padded.  Within tolerance: routing weights and outputs (float32
max-abs 1e-4; bf16 2e-2 x RMS; fp8 6e-2 x RMS of the oracle output).
Small shapes compare every output; the full workload shapes compare every
routing/align result and a sample of output rows."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

SMALL = [
    W.TINY_F32,
    W.MIXTRAL_PREFILL.scaled(name="mixtral_small", M=96, H=256, I=512),
    W.MIXTRAL_PREFILL.scaled(name="mixtral_bm128", M=384, H=128, I=256, E=4),
    W.DECODE_SMALL_EXPERTS.scaled(name="decode_small", M=8, H=256, I=128, E=32, top_k=4),
    W.DEEPSEEK_GROUPED.scaled(name="deepseek_small", M=64, H=256, I=128, E=64),
    W.DEEPSEEK_GROUPED.scaled(name="grouped_softmax_small", M=48, H=128, I=64, E=32,
                              scoring="softmax", renormalize=True, group_count=4, k_group=2,
                              group_select_mode=1, top_k=4, routed_scaling_factor=1.0),
    W.MIXTRAL_PREFILL.scaled(name="contig_fp8_small", M=64, H=256, I=256, weight="fp8"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
@pytest.mark.parametrize("seed_off", [0, 1000, 1001])
def test_small_parity(cfg, seed_off):
    dev = GH.device()
    seed = 1000 + SMALL.index(cfg) + seed_off
    print(f"[case] {cfg.name} seed={seed}", flush=True)
    inp = W.make_inputs(cfg, seed)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, out, ids_o, w_o, what=f"seed{seed}")
    if cfg.out_dtype == "bf16":
        out16, _, _ = GH.run_contiguous(inp, dev)
        GH.check_rounded(out16, out)


def test_tied_integer_logits_route_bit_exact():
    """Integer-valued logits: many exact ties, broken toward the lower index."""
    dev = GH.device()
    for cfg in (W.DEEPSEEK_GROUPED.scaled(name="ties_grouped", M=128, H=64, I=64, E=64),
                W.DECODE_SMALL_EXPERTS.scaled(name="ties_plain", M=128, H=64, I=64, E=128)):
        inp = W.make_inputs(cfg, 77)
        g = torch.Generator().manual_seed(5)
        inp["logits"] = torch.randint(-2, 3, (cfg.M, cfg.E), generator=g).to(torch.bfloat16)
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
        ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        GH.check_output(inp, out, ids_o, w_o, what="ties")


@pytest.mark.parametrize("case", ["one_token", "topk_equals_E", "all_to_one_expert",
                                  "precomputed"])
def test_edge_cases(case):
    dev = GH.device()
    base = W.MIXTRAL_PREFILL.scaled(name=case, M=40, H=128, I=256, E=8)
    if case == "one_token":
        cfg = base.scaled(M=1)
    elif case == "topk_equals_E":
        cfg = base.scaled(E=4, top_k=4)
    else:
        cfg = base
    inp = W.make_inputs(cfg, 31)
    if case in ("all_to_one_expert", "precomputed"):
        rng = np.random.default_rng(3)
        if case == "all_to_one_expert":   # expert 5 takes every first slot, 6 the second
            ids = np.stack([np.full(cfg.M, 5), np.full(cfg.M, 6)], 1).astype(np.int32)
        else:
            ids = np.stack([rng.permutation(cfg.E)[:cfg.top_k] for _ in range(cfg.M)]).astype(
                np.int32)
        w = rng.random((cfg.M, cfg.top_k)).astype(np.float32)
        out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w),
                                          out_dtype=torch.float32)
        GH.check_routing_and_align(inp, ws, info, ids_o=ids, w_o=w.astype(np.float64))
        GH.check_output(inp, out, ids, w.astype(np.float64), what=case)
    else:
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
        ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        GH.check_output(inp, out, ids_o, w_o, what=case)


EDGE_FORMATS = {"fp8": dict(weight="fp8"), "fp8_block": dict(weight="fp8", fp8_block=128),
                "w4z": dict(weight="u4", wq_zero=True), "w8": dict(weight="u8")}


@pytest.mark.parametrize("case", ["one_token", "topk_equals_E", "all_to_one_expert"])
@pytest.mark.parametrize("fmt", list(EDGE_FORMATS))
def test_edge_cases_quantised(case, fmt):
    """The edge cases above on every quantised weight format: a single token,
    top_k = E (every expert active), and all items on two experts (the rest
    empty) against the oracle."""
    dev = GH.device()
    base = W.MIXTRAL_PREFILL.scaled(name=f"{case}_{fmt}", M=40, H=256, I=256, E=8,
                                    **EDGE_FORMATS[fmt])
    cfg = {"one_token": base.scaled(M=1), "topk_equals_E": base.scaled(E=4, top_k=4)}.get(
        case, base)
    inp = W.make_inputs(cfg, 33 + list(EDGE_FORMATS).index(fmt))
    print(f"[case] edge {case} {fmt}", flush=True)
    if case == "all_to_one_expert":
        ids = np.stack([np.full(cfg.M, 5), np.full(cfg.M, 6)], 1).astype(np.int32)
        w = np.random.default_rng(4).random((cfg.M, cfg.top_k)).astype(np.float32)
        out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w),
                                          out_dtype=torch.float32)
        GH.check_routing_and_align(inp, ws, info, ids_o=ids, w_o=w.astype(np.float64))
        GH.check_output(inp, out, ids, w.astype(np.float64), what=f"{case} {fmt}")
    else:
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
        ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        GH.check_output(inp, out, ids_o, w_o, what=f"{case} {fmt}")
    assert B.device_status(ws, info) == 0


def test_inplace_and_deterministic():
    dev = GH.device()
    cfg = W.DEEPSEEK_GROUPED.scaled(name="inplace", M=64, H=256, I=128, E=64)
    inp = W.make_inputs(cfg, 41)
    out1, _, _ = GH.run_contiguous(inp, dev)
    out2, _, _ = GH.run_contiguous(inp, dev)
    assert torch.equal(out1, out2), "two runs differ"
    out3, ws, info = GH.run_contiguous(inp, dev, inplace=True)
    assert torch.equal(out1, out3), "in-place result differs"


def test_precomputed_matches_router_path():
    dev = GH.device()
    cfg = W.DEEPSEEK_GROUPED.scaled(name="pre_vs_router", M=64, H=128, I=128, E=64)
    inp = W.make_inputs(cfg, 43)
    out1, ws, info = GH.run_contiguous(inp, dev)
    K, M = cfg.top_k, cfg.M
    ids = GH.region(ws, info.off_topk_ids, torch.int32, M * K).reshape(M, K)
    w = GH.region(ws, info.off_topk_weights, torch.float32, M * K).reshape(M, K)
    out2, _, _ = GH.run_contiguous(inp, dev, precomputed=(ids, w))
    assert torch.equal(out1, out2)


BATCHED_SMALL = W.BATCHED_FP8.scaled(name="batched_fp8_small", M=96, H=256, I=256, E=8,
                                     top_k=2)


@pytest.mark.parametrize("reduce", [False, True])
def test_batched_fp8_small(reduce):
    dev = GH.device()
    inp = W.make_inputs(BATCHED_SMALL, 1005)
    out, ws, info = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32)
    out16, _, _ = GH.run_batched(inp, dev, reduce=reduce)
    rows, experts = GH.batched_rows(inp)
    if reduce:
        GH.check_rounded(out16, out)
    else:
        flat32 = out.reshape(-1, BATCHED_SMALL.H)[torch.as_tensor(rows, device=out.device)]
        flat16 = out16.reshape(-1, BATCHED_SMALL.H)[torch.as_tensor(rows, device=out.device)]
        GH.check_rounded(flat16, flat32)
    GH.check_batched_tilelist(inp, ws, info)
    import oracle
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=True)
    o_ref, ties = GH.ref_rows(inp, acts, rows, experts)
    if not reduce:
        got = out.float().cpu().numpy().reshape(-1, BATCHED_SMALL.H)[rows]
        GH.compare(BATCHED_SMALL, got, o_ref, "batched rows", ties=ties)
    else:
        y, yties = GH.reduce_rows(inp, rows, o_ref, ties)
        GH.compare(BATCHED_SMALL, out.float().cpu().numpy(), y, "batched reduce", ties=yties)


@pytest.mark.parametrize("weight", ["fp8", "bf16"])
def test_batched_out_alignment(weight):
    """bf16 slab rows are stored as 8-byte pieces when the output is 8-byte
    aligned and one value a lane otherwise: an output view one element past
    an aligned buffer gives the same bits in every valid row, and the rows
    past each expert's count stay as they were."""
    dev = GH.device()
    cfg = BATCHED_SMALL.scaled(name=f"batched_align_{weight}", weight=weight)
    inp = W.make_inputs(cfg, 1007)
    E, T, H = cfg.E, inp["max_tokens"], cfg.H
    print(f"[case] batched output alignment {weight}", flush=True)
    ref, _, _ = GH.run_batched(inp, dev)
    buf = torch.full((E * T * H + 1,), 3.0, dtype=torch.bfloat16, device=dev)
    shifted = buf[1:].view(E, T, H)
    assert shifted.data_ptr() % 8 != 0
    GH.run_batched(inp, dev, out=shifted)
    rows, _ = GH.batched_rows(inp)
    idx = torch.as_tensor(rows, device=dev)
    assert torch.equal(shifted.reshape(-1, H)[idx], ref.reshape(-1, H)[idx])
    untouched = torch.ones(E * T, dtype=torch.bool, device=dev)
    untouched[idx] = False
    assert bool((shifted.reshape(-1, H)[untouched] == 3.0).all())


def test_batched_bf16_matches_contiguous():
    """bf16 batched rows equal the contiguous path's expert rows."""
    dev = GH.device()
    cfg = BATCHED_SMALL.scaled(name="batched_bf16", weight="bf16")
    inp = W.make_inputs(cfg, 1006)
    out, ws, info = GH.run_batched(inp, dev, reduce=True, out_dtype=torch.float32)
    GH.check_batched_tilelist(inp, ws, info)
    import oracle
    rows, experts = GH.batched_rows(inp)
    o_ref, _ = oracle.expert_rows(GH.oracle_experts(inp), oracle.Acts(inp["hidden"].cpu()),
                                  rows, experts)
    pos = {r: i for i, r in enumerate(rows)}
    tmap = inp["token_map"].cpu().numpy()
    wts = inp["token_map_w"].cpu().numpy().astype(np.float64)
    y = np.stack([sum(wts[t, j] * o_ref[pos[tmap[t, j]]] for j in range(cfg.top_k))
                  for t in range(cfg.M)])
    GH.compare(cfg, out.float().cpu().numpy(), y, "batched bf16 reduce")


@pytest.mark.parametrize("tile", ["dma160", "dma160/wc2", "reg64", "reg16", "dma32", "dma64",
                                  "dma256"])
@pytest.mark.parametrize("skew", [False, True])
def test_tile_families_ragged(tile, skew):
    """Every bf16 tile family (160-row DMA ring, 64 / 16-row register-staged,
    32 / 64-row DMA ring) on K and column tails (H % 64 = 16, I % 64 = 48)
    and, with skew, on experts of 200 rows: several row chunks per expert
    and a partial last strip.  "dma160/wc2": the 160-row family with the
    4-wave, 128-column GEMM1 tile instead of the 8-wave one small problems
    get."""
    dev = GH.device()
    hint = GH.tile_kwargs(tile)
    cfg = W.MIXTRAL_PREFILL.scaled(name=f"ragged_{tile}", M=200, H=208, I=176, E=4)
    inp = W.make_inputs(cfg, 51)
    print(f"[case] ragged tile={tile} skew={skew}", flush=True)
    if skew:
        ids = np.stack([np.full(cfg.M, 1), np.full(cfg.M, 2)], 1).astype(np.int32)
        w = np.random.default_rng(4).random((cfg.M, cfg.top_k)).astype(np.float32)
        out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w), out_dtype=torch.float32,
                                          **hint)
        GH.check_routing_and_align(inp, ws, info, ids_o=ids, w_o=w.astype(np.float64))
        GH.check_output(inp, out, ids, w.astype(np.float64), what="ragged skew")
    else:
        out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, **hint)
        ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
        GH.check_output(inp, out, ids_o, w_o, what="ragged")
    out16, _, _ = GH.run_contiguous(inp, dev, precomputed=(ids, w) if skew else None, **hint)
    GH.check_rounded(out16, out)


@pytest.mark.parametrize("packed", [False, True])
def test_gemm2_k_split(packed):
    """The 160-row family on a problem whose GEMM2 runs as two K halves
    (I >= 1024, few tiles): I = 1040 also leaves a K tail in the second half,
    and biases check that b2 enters once."""
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name="k_split", M=96, H=256, I=1040, E=4, bias=True)
    inp = W.make_inputs(cfg, 71)
    print(f"[case] gemm2 k split packed={packed}", flush=True)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=packed,
                                      **GH.tile_kwargs("dma160"))
    assert info.off_o2 != 0, "the second GEMM did not run split in K"
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, out, ids_o, w_o, what="k split")


# Routing / align launch shapes, with tiny expert FFNs so the oracle stays
# fast: (M, E, top_k, scoring, groups).  Lanes per token: 8, 16, 32 or 64
# (E <= 64), several experts per lane above 64.  Past 8192 routed items the
# align streams its items through LDS in batches; at E = 1024 its LDS passes
# 64 KiB.
ROUTE_PATHS = [
    ("lpt8", 200, 8, 2, "softmax", 1),
    ("lpt16", 96, 16, 3, "sigmoid", 1),
    ("lpt32_tail", 70, 24, 5, "softmax", 1),
    ("e1024_lds_over_64k", 6, 1024, 8, "softmax", 1),
    ("lpt8_many_tokens", 1500, 8, 2, "softmax", 1),
    ("lpt16_multibatch", 3000, 16, 4, "softmax", 1),
    ("e256_grouped_multibatch", 1300, 256, 8, "sigmoid", 8),
    ("e512", 300, 512, 6, "softmax", 1),
    # grouped keys from LDS: 12 experts a group over 6 lanes (not a power of two)
    ("e96_groups_of_12", 400, 96, 6, "sigmoid", 8),
    # grouped keys by shuffles over 8-lane groups, softmax top-2 sums, 4 of 6 groups
    ("e192_six_groups", 400, 192, 6, "softmax", 6),
    # the largest top_k (32) the boundary takes, over the most experts (1024)
    ("topk32_e1024", 40, 1024, 32, "softmax", 1),
    # top_k = 32 = k_group x experts a group: every expert of the 4 chosen groups
    ("topk32_grouped_e64", 64, 64, 32, "sigmoid", 8),
]


@pytest.mark.parametrize("case", ROUTE_PATHS, ids=[c[0] for c in ROUTE_PATHS])
def test_route_align_paths(case):
    name, M, E, K, scoring, G = case
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name=name, M=M, H=32, I=32, E=E, top_k=K, scoring=scoring,
                                   renormalize=scoring == "softmax", group_count=G,
                                   k_group=min(G, 4), group_select_mode=1 if G > 1 else 0,
                                   routed_scaling_factor=1.5 if G > 1 else 1.0)
    print(f"[case] route/align {name} M={M} E={E} k={K}", flush=True)
    inp = W.make_inputs(cfg, 2000 + ROUTE_PATHS.index(case))
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    tokens = None if M <= 64 else np.arange(0, M, max(1, M // 48))
    GH.check_output(inp, out, ids_o, w_o, tokens=tokens, what=name)


@pytest.mark.parametrize("H", [208, 2304])
def test_fp8_activation_codes_bit_exact(H):
    """The in-path per-token fp8 quantisation (scale = amax / 448, RNE,
    saturating) produces the oracle's codes and scales bit for bit: contiguous
    rows by token, batched rows at their padded positions.  Rows of up to 2048
    bf16 columns are coded from registers, longer ones in a second pass."""
    import oracle
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name="contig_fp8_codes", M=96, H=H, I=256, weight="fp8")
    inp = W.make_inputs(cfg, 81)
    inp["hidden"][3] = 0.0                         # an all-zero row: scale 1, codes 0
    _, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    q_ref, s_ref = oracle.quant_rows_fp8(inp["hidden"].float().numpy())
    q = GH.region(ws, info.off_aq, torch.uint8, cfg.M * cfg.H).reshape(cfg.M, cfg.H)
    s = GH.region(ws, info.off_aq_scale, torch.float32, cfg.M)
    assert np.array_equal(q, q_ref.reshape(cfg.M, cfg.H))
    assert np.array_equal(s.view(np.uint32), np.asarray(s_ref, np.float32).view(np.uint32))

    inp = W.make_inputs(BATCHED_SMALL, 1008)
    _, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32)
    T, H, BM = inp["max_tokens"], BATCHED_SMALL.H, info.block_m
    counts = inp["expert_num_tokens"].cpu().numpy()
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    q = GH.region(ws, info.off_aq, torch.uint8, npp * H).reshape(npp, H)
    s = GH.region(ws, info.off_aq_scale, torch.float32, npp)
    xb = inp["hidden"].float().numpy().reshape(-1, H)
    p = 0
    for e, c in enumerate(counts):
        if c:
            q_ref, s_ref = oracle.quant_rows_fp8(xb[e * T:e * T + c])
            assert np.array_equal(q[p:p + c], q_ref.reshape(c, H)), e
            assert np.array_equal(s[p:p + c], np.asarray(s_ref, np.float32)), e
        p += -(-c // BM) * BM


@pytest.mark.parametrize("weight", ["bf16", "fp8"])
def test_empty_inputs(weight):
    """No tokens: a contiguous forward with M = 0 returns at once, and batched
    slabs whose expert_num_tokens are all zero leave every slab row as it was
    (no tile is computed)."""
    dev = GH.device()
    E, H, I, T = 8, 128, 256, 32
    cfg = W.MIXTRAL_PREFILL.scaled(name=f"empty_{weight}", M=0, H=H, I=I, E=E, weight=weight)
    print(f"[case] empty contiguous {weight}", flush=True)
    inp = W.make_inputs(cfg.scaled(M=4), 51)          # weights; the token arrays are cut to 0
    w13, w2 = inp["w13"].to(dev), inp["w2"].to(dev)
    kw = {k: inp[k].to(dev) for k in ("w13_scale", "w2_scale") if inp.get(k) is not None}
    hidden = torch.zeros(0, H, dtype=torch.bfloat16, device=dev)
    logits = torch.zeros(0, E, dtype=torch.bfloat16, device=dev)
    out, ws, info = B.fused_moe(hidden, w13, w2, logits, top_k=2, **kw)
    torch.cuda.synchronize()
    assert out.shape == (0, H)

    print(f"[case] empty batched slabs {weight}", flush=True)
    slabs = torch.randn(E, T, H, device=dev).to(torch.bfloat16)
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    sentinel = torch.full((E, T, H), 7.0, dtype=torch.bfloat16, device=dev)
    out = sentinel.clone()
    B.fused_moe_batched(slabs, counts, w13, w2, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel), "an empty expert's slab rows were written"
