"""The fp8 path's re-quantised intermediate z read back from the workspace
and compared with the oracle code by code (FlagGems walkthrough, "FP8 W8A8":
the intermediate is quantised again before the second GEMM; here per row and
128 columns), for every routed item's padded row of z and its group scales.

The device forms h in float32 from fp32 MFMA accumulators, the oracle in
float64, and where h is the small difference of large products (h_gate near
zero, say) their z differ by more than any relative window around a rounding
tie.  So the bar is: the group scales within SCALE_RTOL of the oracle's; every
code the oracle's, or one fp8 step from it (plus ABS_TOL in code units for
the subnormal codes of values below about 3e-5 of the group's amax); and at
most MAX_DIFF_FRAC of all codes (MAX_ITEM_FRAC of one item's) differing.  A
wrong column, row, group, scale, bias or gate / up order moves most codes by
many steps and fails it.  The oracle's near-tie report (TIE_WINDOW) is
printed beside the count of differing codes."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE_RTOL = 2e-4
ABS_TOL = 0.01
MAX_DIFF_FRAC = 0.01
MAX_ITEM_FRAC = 0.05


def _decode(c):
    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()


def _step(v):
    """The fp8 E4M3FN spacing at magnitude v (2^-9 below the normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    return 2.0 ** (e - 3)


def _compare(cfg, ws, info, rows, experts, positions, inp, acts, what):
    """Device z codes / scales at `positions` against the oracle's for
    (activation row, expert) pairs (rows, experts)."""
    I = cfg.I
    G = I // 128
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    zall = GH.region(ws, info.off_z, torch.uint8, npp * I).reshape(npp, I)
    zs_ld = info.max_sorted_len + 256                    # group-major [I/128][zs_ld]
    sall = GH.region(ws, info.off_z_scale, torch.float32, G * zs_ld).reshape(G, zs_ld)
    codes, scales, alt = oracle.expert_z_codes(GH.oracle_experts(inp), acts, rows, experts,
                                               tie_window=GH.TIE_WINDOW)
    got = zall[positions]
    got_s = sall[:, positions].T
    srel = np.abs(got_s.astype(np.float64) / scales - 1.0).max()
    assert srel <= SCALE_RTOL, f"{what}: z scales differ by {srel:.2e} relative"
    t_or, t_dev = _decode(codes), _decode(got)
    diff = got != codes
    far = np.abs(t_dev - t_or) > _step(np.maximum(np.abs(t_or), np.abs(t_dev))) + ABS_TOL
    ties = int((diff & (alt >= 0) & (got.astype(np.int16) == alt)).sum())
    print(f"[zcodes] {what}: {got.size} codes, {int(diff.sum())} differ ({ties} of them at "
          f"reported near-ties, {int((alt >= 0).sum())} reported), scale rel {srel:.1e}",
          flush=True)
    bad = np.argwhere(far)
    assert bad.size == 0, (f"{what}: {len(bad)} z codes more than a step off, first (item, "
                           f"column) {bad[:5].tolist()}")
    assert diff.mean() <= MAX_DIFF_FRAC, f"{what}: {diff.mean():.3%} of the codes differ"
    worst = diff.mean(axis=1).max()
    assert worst <= MAX_ITEM_FRAC, f"{what}: {worst:.3%} of one item's codes differ"


CONTIG = [
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_fp8", M=96, H=256, I=384, E=8, top_k=2,
                              weight="fp8", bias=True), False),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_fp8_packed", M=300, H=208, I=256, E=4, top_k=2,
                              weight="fp8", bias=True), True),
    (W.MIXTRAL_PREFILL.scaled(name="z_contig_blockfp8", M=80, H=384, I=256, E=8, top_k=2,
                              weight="fp8", fp8_block=128), True),
]


@pytest.mark.parametrize("case", CONTIG, ids=[c[0].name for c in CONTIG])
def test_z_codes_contiguous(case):
    cfg, packed = case
    dev = GH.device()
    print(f"[case] z codes {cfg.name} packed={packed}", flush=True)
    inp = W.make_inputs(cfg, 4100 + CONTIG.index(case))
    _, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=packed)
    ids_o, _ = GH.check_routing_and_align(inp, ws, info)
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    sorted_ids = GH.region(ws, info.off_sorted_ids, torch.int32, npp)
    pos = np.nonzero(sorted_ids < cfg.M * cfg.top_k)[0]
    r = sorted_ids[pos]
    tokens, experts = r // cfg.top_k, ids_o.reshape(-1)[r]
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=True, block=cfg.fp8_block)
    _compare(cfg, ws, info, tokens, experts, pos, inp, acts, cfg.name)


def test_z_codes_batched_skewed():
    """Batched slabs, one expert past two 128-row tiles, packed weights."""
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="z_batched_fp8", M=400, H=256, I=384, E=4, top_k=2)
    inp = W.make_inputs(cfg, 4200)
    counts = inp["expert_num_tokens"].cpu().numpy()
    print(f"[case] z codes batched counts={counts.tolist()}", flush=True)
    assert counts.max() > 256
    _, ws, info = GH.run_batched(inp, dev, reduce=False, out_dtype=torch.float32, packed=True)
    GH.check_batched_tilelist(inp, ws, info)
    npp = int(GH.region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    sorted_ids = GH.region(ws, info.off_sorted_ids, torch.int32, npp)
    T = inp["max_tokens"]
    pos = np.nonzero(sorted_ids < cfg.E * T)[0]
    rows = sorted_ids[pos].astype(np.int64)
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=True, block=cfg.fp8_block)
    _compare(cfg, ws, info, rows, rows // T, pos, inp, acts, cfg.name)
