"""Packed weight layouts (moe_pack_weights, bf16 and fp8): the packed bytes
follow the layouts moe.h documents, and a forward on packed weights equals
the forward on the plain weights bit for bit (same products, same summation
order) and so meets the oracle bar wherever the plain path does."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu


def _swz(k):
    return 2 * ((k & 3) | ((k >> 1) & 4))


def _ref_pack(w, gate_up):
    """The documented layout, written out with numpy: 16 KiB blocks of 64 rows
    x 16 slots of 8 columns; slot s of row k holds chunk s ^ swz(k)."""
    E, K, N = w.shape
    ncols = N // 2 if gate_up else N          # columns per half (w13) / all (w2)
    bw = 64 if gate_up else 128               # columns of one half-block / block
    nblk, nks = -(-ncols // bw), -(-K // 64)
    out = np.zeros((E, nks, nblk, 64, 16, 8), dtype=np.uint16)
    for j in range(nblk):
        for kt in range(nks):
            for k in range(64):
                row = kt * 64 + k
                if row >= K:
                    continue
                for s in range(16):
                    c = s ^ _swz(k)
                    if gate_up:
                        col = bw * j + 8 * (c % 8)
                        if col >= ncols:
                            continue
                        src = col if c < 8 else ncols + col
                    else:
                        src = bw * j + 8 * c
                        if src >= ncols:
                            continue
                    out[:, kt, j, k, s, :] = w[:, row, src:src + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("E,H,I", [(2, 208, 176), (3, 128, 256)])
def test_pack_layout_bytes(E, H, I):
    dev = GH.device()
    g = torch.Generator().manual_seed(7)
    w13 = torch.randn(E, H, 2 * I, generator=g).to(torch.bfloat16)
    w2 = torch.randn(E, I, H, generator=g).to(torch.bfloat16)
    print(f"[case] pack E={E} H={H} I={I}", flush=True)
    pw = B.pack_weights(w13.to(dev), w2.to(dev))
    torch.cuda.synchronize()
    got13 = pw.w13.cpu().view(torch.int16).numpy().view(np.uint16)
    got2 = pw.w2.cpu().view(torch.int16).numpy().view(np.uint16)
    ref13 = _ref_pack(w13.view(torch.int16).numpy().view(np.uint16), True)
    ref2 = _ref_pack(w2.view(torch.int16).numpy().view(np.uint16), False)
    assert got13.shape == ref13.shape and got2.shape == ref2.shape
    assert np.array_equal(got13, ref13)
    assert np.array_equal(got2, ref2)


SMALL_BF16 = [
    W.MIXTRAL_PREFILL.scaled(name="mixtral_small", M=96, H=256, I=512),
    W.MIXTRAL_PREFILL.scaled(name="mixtral_bm128", M=384, H=128, I=256, E=4),
    W.DECODE_SMALL_EXPERTS.scaled(name="decode_small", M=8, H=256, I=128, E=32, top_k=4),
    W.DEEPSEEK_GROUPED.scaled(name="deepseek_small", M=64, H=256, I=128, E=64),
    W.MIXTRAL_PREFILL.scaled(name="ragged", M=200, H=208, I=176, E=4),
]


@pytest.mark.parametrize("tile", ["auto", "dma160", "dma160/wc2", "reg64", "reg16", "dma256"])
@pytest.mark.parametrize("cfg", SMALL_BF16, ids=[c.name for c in SMALL_BF16])
def test_packed_equals_plain_small(cfg, tile):
    dev = GH.device()
    hint = GH.tile_kwargs(tile)
    inp = W.make_inputs(cfg, 61)
    print(f"[case] packed {cfg.name} tile={tile}", flush=True)
    plain, _, _ = GH.run_contiguous(inp, dev, out_dtype=torch.float32, **hint)
    packed, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=True, **hint)
    assert torch.equal(plain, packed)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, packed, ids_o, w_o, what="packed")


@pytest.mark.parametrize("cfg", [W.MIXTRAL_PREFILL, W.DEEPSEEK_GROUPED],
                         ids=["mixtral_prefill_bf16", "deepseek_grouped_sigmoid_bf16"])
def test_packed_equals_plain_full_size(cfg):
    dev = GH.device()
    inp = W.make_inputs(cfg, 1000 + W.CONFIGS.index(cfg), device=dev)
    print(f"[case] packed full {cfg.name}", flush=True)
    plain, _, _ = GH.run_contiguous(inp, dev)
    packed, _, _ = GH.run_contiguous(inp, dev, packed=True)
    assert torch.equal(plain, packed)


def test_packed_batched_bf16():
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="batched_bf16_packed", M=96, H=256, I=256, E=8,
                               weight="bf16")
    inp = W.make_inputs(cfg, 1006)
    for reduce in (False, True):
        plain, _, _ = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32)
        packed, _, _ = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32,
                                      packed=True)
        rows, _ = GH.batched_rows(inp) if not reduce else (None, None)
        if reduce:
            assert torch.equal(plain, packed)
        else:
            idx = torch.as_tensor(rows, device=dev)
            flat_p, flat_k = plain.reshape(-1, cfg.H)[idx], packed.reshape(-1, cfg.H)[idx]
            assert torch.equal(flat_p, flat_k)


def _ref_pack_f8(w, gate_up):
    """The documented fp8 layout, written out with numpy: 16 KiB blocks of 128
    columns x 128 K bytes; column c's 16-byte slot s holds K chunk 2 (p & 3) + (p >> 2),
    p = s ^ ((c >> 1) & 7).  w13 halves: block column 32 h + 16 f + s of a half
    is the half's column 32 h + 2 s + f."""
    E, K, N = w.shape
    half = N // 2
    nblk = half // 64 if gate_up else -(-N // 128)
    nks = -(-K // 128)
    out = np.zeros((E, nks, nblk, 128, 8, 16), dtype=np.uint8)
    for j in range(nblk):
        for c in range(128):
            if gate_up:
                h = c % 64
                pc = 32 * (h // 32) + 2 * (h % 16) + (h % 32) // 16
                col = 64 * j + pc if c < 64 else half + 64 * j + pc
            else:
                col = 128 * j + c
                if col >= N:
                    continue
            for kt in range(nks):
                for sl in range(8):
                    p = sl ^ ((c >> 1) & 7)
                    chunk = 2 * (p & 3) + (p >> 2)
                    rows = kt * 128 + chunk * 16 + np.arange(16)
                    ok = rows < K
                    out[:, kt, j, c, sl, :ok.sum()] = w[:, rows[ok], col]
    return out.reshape(-1)


@pytest.mark.parametrize("E,H,I", [(2, 208, 256), (3, 128, 384)])
def test_pack_layout_bytes_fp8(E, H, I):
    dev = GH.device()
    g = torch.Generator().manual_seed(9)
    w13 = (torch.randn(E, H, 2 * I, generator=g) * 8).to(torch.float8_e4m3fn)
    w2 = (torch.randn(E, I, H, generator=g) * 8).to(torch.float8_e4m3fn)
    print(f"[case] pack fp8 E={E} H={H} I={I}", flush=True)
    pw = B.pack_weights(w13.to(dev), w2.to(dev))
    torch.cuda.synchronize()
    got13, got2 = pw.w13.cpu().numpy(), pw.w2.cpu().numpy()
    ref13 = _ref_pack_f8(w13.view(torch.uint8).numpy(), True)
    ref2 = _ref_pack_f8(w2.view(torch.uint8).numpy(), False)
    assert got13.shape == ref13.shape and got2.shape == ref2.shape
    assert np.array_equal(got13, ref13)
    assert np.array_equal(got2, ref2)


# fp8: packed weights run the 256-row LDS-DMA kernels, plain weights the
# register-staged ones; both sum the same products in the same order.
FP8_CASES = [
    W.MIXTRAL_PREFILL.scaled(name="contig_fp8_small", M=64, H=256, I=256, weight="fp8"),
    W.MIXTRAL_PREFILL.scaled(name="contig_fp8_ragged_bias", M=300, H=208, I=384, E=4,
                             weight="fp8", bias=True),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=[c.name for c in FP8_CASES])
def test_packed_fp8_equals_plain_contiguous(cfg):
    dev = GH.device()
    inp = W.make_inputs(cfg, 63)
    print(f"[case] packed fp8 {cfg.name}", flush=True)
    plain, _, _ = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    packed, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=True)
    assert torch.equal(plain, packed)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, packed, ids_o, w_o, what="packed fp8")


@pytest.mark.parametrize("reduce", [False, True])
def test_packed_fp8_batched_skewed(reduce):
    """Batched fp8 with expert runs past one 256-row tile, a K tail in GEMM1
    (H % 128 = 80) and a column tail in GEMM2 (H < 256)."""
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="batched_fp8_skew_packed", M=400, H=208, I=384, E=4,
                               top_k=2)
    inp = W.make_inputs(cfg, 1007)
    counts = inp["expert_num_tokens"].cpu().numpy()
    print(f"[case] packed fp8 batched reduce={reduce} counts={counts.tolist()}", flush=True)
    assert counts.max() > 256
    plain, _, _ = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32)
    packed, ws, info = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32,
                                      packed=True)
    rows, experts = GH.batched_rows(inp)
    if reduce:
        assert torch.equal(plain, packed)
    else:
        idx = torch.as_tensor(rows, device=dev)
        assert torch.equal(plain.reshape(-1, cfg.H)[idx], packed.reshape(-1, cfg.H)[idx])
        import oracle
        acts = oracle.Acts(inp["hidden"].cpu(), quantize=True)
        o_ref, ties = GH.ref_rows(inp, acts, rows, experts)
        got = packed.reshape(-1, cfg.H)[idx].cpu().numpy()
        GH.compare(cfg, got, o_ref, "packed fp8 batched rows", ties=ties)


def test_wide_tiles_mixed_chunk_counts():
    """About 128 rows per expert on average (the 256-column GEMM tiles) with
    skewed experts: single-chunk experts stream their weights with the
    non-temporal policy, multi-chunk ones share them; plain and packed
    weights agree bit for bit and meet the oracle bar."""
    dev = GH.device()
    cfg = W.DEEPSEEK_GROUPED.scaled(name="wide_mixed_chunks", M=256, H=256, I=384, E=16, top_k=8,
                                    group_count=4, k_group=2)
    inp = W.make_inputs(cfg, 1011)
    print(f"[case] {cfg.name}", flush=True)
    plain, _, _ = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    packed, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=True)
    counts = GH.region(ws, info.off_expert_counts, torch.int32, cfg.E)
    assert counts.sum() <= cfg.E * 160 and counts.max() > 160, counts
    assert torch.equal(plain, packed)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, packed, ids_o, w_o, what="wide tiles, mixed chunks")
