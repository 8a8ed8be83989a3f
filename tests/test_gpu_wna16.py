"""WNA16 (8- and 4-bit weight codes with group scales and zero points, bf16
activations) against the CPU oracle, and the packed code layout bit for bit.

Outputs within the bf16 bound (2e-2 x RMS of the oracle's double result),
against the oracle fed the weights the path computes with: the exact
dequantised weights (small-row tiles) or those weights in bf16 (the 160-row
tile); gpu_harness.Readings holds both and the closer one is taken.  Routing
and align bit for bit as everywhere else."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

WQ_SMALL = [
    # a few rows per expert (32-row tiles), short last K group (H 320)
    W.DECODE_SMALL_EXPERTS.scaled(name="w4_decode", M=8, H=320, I=256, E=32, top_k=4,
                                  weight="u4"),
    W.DECODE_SMALL_EXPERTS.scaled(name="w8z_decode", M=8, H=320, I=256, E=32, top_k=4,
                                  weight="u8", wq_zero=True),
    # about 16 rows per expert (64-row tiles), zero points, biases
    W.MIXTRAL_PREFILL.scaled(name="w4z_mid", M=64, H=256, I=384, E=8, weight="u4",
                             wq_zero=True, bias=True),
    # 256 rows per expert (160-row tiles, two chunks), grouped sigmoid routing
    W.DEEPSEEK_GROUPED.scaled(name="w8_prefill", M=512, H=256, I=256, E=8, top_k=4,
                              group_count=4, k_group=2, weight="u8"),
    # scale groups of 32 and 64 K rows (GPTQ / AWQ group sizes) on every tile
    # family; H 352 and I 272 leave short last groups and a stage whose second
    # 32-row group is past K
    W.DECODE_SMALL_EXPERTS.scaled(name="w4z_g32_decode", M=8, H=352, I=272, E=32, top_k=4,
                                  weight="u4", wq_zero=True, wq_group=32),
    W.DECODE_SMALL_EXPERTS.scaled(name="w8_g64_decode", M=8, H=352, I=272, E=32, top_k=4,
                                  weight="u8", wq_group=64),
    W.MIXTRAL_PREFILL.scaled(name="w8z_g32_mid", M=64, H=256, I=384, E=8, weight="u8",
                             wq_zero=True, bias=True, wq_group=32),
    W.MIXTRAL_PREFILL.scaled(name="w4_g64_mid", M=64, H=256, I=384, E=8, weight="u4",
                             wq_group=64),
    W.DEEPSEEK_GROUPED.scaled(name="w4z_g32_prefill", M=512, H=352, I=272, E=8, top_k=4,
                              group_count=4, k_group=2, weight="u4", wq_zero=True, wq_group=32),
    W.DEEPSEEK_GROUPED.scaled(name="w8z_g64_prefill", M=512, H=256, I=256, E=8, top_k=4,
                              group_count=4, k_group=2, weight="u8", wq_zero=True, wq_group=64),
]


@pytest.mark.parametrize("cfg", WQ_SMALL, ids=[c.name for c in WQ_SMALL])
@pytest.mark.parametrize("seed_off", [0, 1000])
def test_wna16_small_parity(cfg, seed_off):
    dev = GH.device()
    seed = 4000 + WQ_SMALL.index(cfg) + seed_off
    print(f"[case] {cfg.name} seed={seed}", flush=True)
    inp = W.make_inputs(cfg, seed)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, out, ids_o, w_o, what=f"seed{seed}")
    out16, _, _ = GH.run_contiguous(inp, dev)
    GH.check_rounded(out16, out)


def test_wna16_batched():
    """Batched slabs with 4-bit codes and zero points (rows past the counts
    are NaN and never reach valid rows)."""
    import oracle
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="w4_batched", M=96, H=256, I=256, E=8, top_k=2, weight="u4",
                               wq_zero=True)
    inp = W.make_inputs(cfg, 4100)
    out, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32)
    GH.check_batched_tilelist(inp, ws, info)
    rows, experts = GH.batched_rows(inp)
    ref, alt = GH.ref_rows(inp, oracle.Acts(inp["hidden"].cpu()), rows, experts)
    got = out.reshape(-1, cfg.H)[torch.as_tensor(rows, device=out.device)]
    GH.compare(cfg, got.cpu().numpy(), ref, "batched w4", ties=alt)


def _fragment_order(codes, bits, w13, H, I):
    """numpy reference of the documented packed order: blocks (e, kt, j) of
    128 columns x 64 K rows; lane group ((2 f + h) * 64 + l) holds column
    16 f + l % 16 and K rows 64 kt + 32 h + 8 (l // 16) + 0..7 (8-bit: one
    byte each; 4-bit: row i of the eight in nibble i // 2 + 4 (i % 2))."""
    c = codes.astype(np.int64)
    if bits == 4:
        c = np.stack([c & 15, c >> 4], -1).reshape(*c.shape[:-1], -1)
    E, K, N = c.shape
    nks = -(-K // 64)
    nblk = -(-I // 64) if w13 else -(-H // 128)
    out = []
    for e in range(E):
        for kt in range(nks):
            for j in range(nblk):
                blk = np.zeros((8, 2, 64, 8), np.int64)
                for f in range(8):
                    for h in range(2):
                        for l in range(64):
                            bc = 16 * f + l % 16
                            if w13:
                                zc = 64 * j + bc % 64
                                col, ok = (zc if bc < 64 else I + zc), zc < I
                            else:
                                col = 128 * j + bc
                                ok = col < H
                            for i in range(8):
                                k = 64 * kt + 32 * h + 8 * (l // 16) + i
                                if ok and k < K:
                                    blk[f, h, l, i] = c[e, k, col]
                out.append(blk.reshape(-1, 8))
    v = np.concatenate(out)
    if bits == 8:
        return v.astype(np.uint8).ravel()
    # 4-bit: code i in nibble i // 2 + 4 * (i % 2) of the lane's 32-bit word
    word = np.zeros(v.shape[0], np.int64)
    for i in range(8):
        word |= v[:, i] << (4 * (i // 2 + 4 * (i % 2)))
    return word.astype("<u4").view(np.uint8).ravel()


@pytest.mark.parametrize("bits", [8, 4])
def test_wna16_pack_layout(bits):
    dev = GH.device()
    E, H, I = 2, 80, 96                 # partial blocks in K and N
    g = torch.Generator().manual_seed(bits)
    hi = 256 if bits == 8 else 16
    q13 = torch.randint(0, hi, (E, H, 2 * I), generator=g, dtype=torch.int64)
    q2 = torch.randint(0, hi, (E, I, H), generator=g, dtype=torch.int64)

    def store(q):
        q = q.to(torch.uint8)
        return q if bits == 8 else (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    w13, w2 = store(q13), store(q2)
    pw = B.pack_weights(w13.to(dev), w2.to(dev), wq_bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(pw.w13.cpu().numpy(), _fragment_order(w13.numpy(), bits, True, H, I))
    assert np.array_equal(pw.w2.cpu().numpy(), _fragment_order(w2.numpy(), bits, False, H, I))


@pytest.mark.parametrize("name", ["decode_e128_w4a16", "decode_e128_w8a16"])
def test_wna16_full_size_decode(name):
    cfg = W.BY_NAME[name]
    dev = GH.device()
    seed = 1100 + W.EXTRA.index(cfg)
    print(f"[case] {cfg.name} seed={seed}", flush=True)
    inp = W.make_inputs(cfg, seed, device=dev)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_z_all_contiguous(inp, ws, info, ids_o, dev, "full wna16, every item's z")
    GH.check_output(inp, out, ids_o, w_o, what="full wna16")


# GPTQ / AWQ checkpoints: int32 code words -> moe_repack_wna16 -> the packed
# layout -> the forward, against the oracle's own unpacking of the same words.
CHECKPOINTS = [("gptq", 4, 128, True, 1), ("gptq", 4, 32, False, 0), ("gptq", 8, 64, True, 1),
               ("awq", 4, 128, True, 0), ("awq", 4, 64, True, 0), ("awq", 4, 32, False, 0)]


@pytest.mark.parametrize("fmt,bits,G,zero,adjust", CHECKPOINTS,
                         ids=[f"{c[0]}{c[1]}_g{c[2]}{'_z' if c[3] else ''}" for c in CHECKPOINTS])
def test_checkpoint_codes_repacked(fmt, bits, G, zero, adjust):
    """Codes and zero points of a synthetic checkpoint (the workload
    generator's packers write GPTQ / AWQ words; GPTQ with adjust 1 stores
    z - 1) re-packed on the device equal the oracle's unpacking bit for bit,
    and the forward on them meets the oracle's bar."""
    import oracle
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name=f"ckpt_{fmt}{bits}_g{G}", M=48, H=256, I=320, E=8,
                                   weight=f"u{bits}", wq_zero=zero, wq_group=G)
    inp = W.make_inputs(cfg, 4200 + bits + G)
    words = {}
    for name in ("w13", "w2"):
        q = inp[name]
        if bits == 4:                                   # one code a byte for the packer
            q = torch.stack([q & 15, q >> 4], -1).reshape(*q.shape[:-1], -1)
        z = inp[f"{name}_zero"]
        stored = None if z is None else ((z.to(torch.int64) - adjust) % (1 << bits)).to(
            torch.uint8)
        words[name] = W.pack_wq_checkpoint(q, stored, bits, fmt)
    print(f"[case] checkpoint {fmt} bits={bits} group={G} zero={zero}", flush=True)
    for name, (K, N) in (("w13", (cfg.H, 2 * cfg.I)), ("w2", (cfg.I, cfg.H))):
        qw, qz = words[name]
        codes, zeros = B.repack_wna16(fmt, bits, qw.to(dev), None if qz is None else qz.to(dev),
                                      K=K, N=N, group=G, zero_adjust=adjust)
        ref_c, ref_z = oracle.unpack_wq(fmt, bits, qw, qzeros=qz, K=K, N=N, group=G,
                                        zero_adjust=adjust)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), ref_c), name
        assert np.array_equal(inp[name].numpy(), ref_c), name      # the generator's codes
        if zero:
            assert np.array_equal(zeros.cpu().numpy(), ref_z), name
            assert np.array_equal(inp[f"{name}_zero"].numpy(), ref_z), name
        inp[name] = torch.from_numpy(ref_c)
        if zero:
            inp[f"{name}_zero"] = torch.from_numpy(ref_z)
    out, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32)
    ids_o, w_o = GH.check_routing_and_align(inp, ws, info)
    GH.check_output(inp, out, ids_o, w_o, what=f"{fmt} checkpoint")
