"""Shared helpers of the GPU tests: run the HIP path through the C ABI on
seeded inputs, read its intermediates back from the workspace, and check
them and the output against the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

# Output tolerances: max |gpu - oracle| over the checked outputs, against the
# oracle's unrounded (double) result.  float32 absolute; bf16 and fp8
# relative to the RMS of the oracle output.  The bound applies to the
# computed result, which the path can hand out in float32; its bf16 output is
# that float32 result rounded once to nearest-even (checked bit for bit), so a
# bf16 output may differ from the oracle by the bound plus half a bf16 ulp --
# storage rounding that on its own exceeds 2e-2 x RMS wherever |y| > 5.12 RMS.
TOL_F32_ABS = 1e-4
TOL_BF16_RMS = 2e-2
TOL_FP8_RMS = 6e-2
TOL_WEIGHT = 1e-5          # routing weights, relative to max(1, routed_scaling_factor)
# fp8 z requantisation: the device's z differs from the oracle's in its last
# bits (float32 sums in another order, hardware exp / reciprocal), so a z code
# whose z / scale lies within this relative distance of a rounding midpoint
# may be rounded either way, and both outputs are correct.  The oracle reports
# such codes with the output change of each flip; compare() measures the
# error against the closest of those equally correct references.
TIE_WINDOW = 1e-4
# WNA16 (u8 / u4 codes, bf16 activations) is held to the bf16 bound, against
# the oracle fed the weights the path computes with.  The walkthrough's entry
# point dequantises the codes to hidden_states.dtype (bf16) before its
# generic kernel runs; the 160-row tile does the same, while the small-row
# tiles compute more exactly (raw codes into the MFMAs, scale and zero point
# applied per group), i.e. with the exact weight (q - z) s.  So an output is
# compared with the oracle under both readings and held to the bound against
# the closer one (Readings).
WQ_BITS = {"u8": 8, "u4": 4}
# z, the intermediate the first GEMM writes, read back from the workspace and
# compared with the oracle's z (before any requantisation).  float32 / bf16 z:
# within Z_REL of its own magnitude (bf16: one ulp, 2^-7 at the start of a
# binade; the storage rounding takes up to half of it, and a z the device
# forms in float32 next to a rounding midpoint may round to the other
# neighbour) plus Z_RMS of its row's RMS (the device sums the products in
# float32, and where they cancel h keeps only their absolute error).  fp8 z:
# see check_z_codes.  WNA16 z: the same bound, against the closer of the two
# readings of its weights.
Z_REL = {2: 2.0 ** -7, 4: 1e-5}
Z_RMS = 1e-3
# fp8 z: the group scales within Z_SCALE_RTOL; every code the oracle's or one
# E4M3FN step from it (plus Z_ABS_TOL in code units, for the subnormal codes
# of values below about 3e-5 of the group's amax), and at most Z_MAX_FRAC of
# all codes (Z_MAX_ITEM_FRAC of one item's) differing.  A wrong column, row,
# group, scale, bias or gate / up order moves most codes by many steps.
Z_SCALE_RTOL = 2e-4
Z_ABS_TOL = 0.01
Z_MAX_FRAC = 0.01
Z_MAX_ITEM_FRAC = 0.05


# Named tile families for the tests (moe_problem.tile_hint / gemm1_wave_cols).
TILES = {"auto": B.MOE_TILE_AUTO, "dma160": B.MOE_TILE_DMA_160, "reg64": B.MOE_TILE_REG_64,
         "reg16": B.MOE_TILE_REG_16, "dma32": B.MOE_TILE_DMA_32, "dma64": B.MOE_TILE_DMA_64,
         "dma256": B.MOE_TILE_DMA_256}


def tile_kwargs(name: str) -> dict:
    """fused_moe keyword arguments forcing a tile family: "dma160", or
    "dma160/wc2" for that family with the 128-column GEMM1 tile."""
    fam, _, wc = name.partition("/wc")
    kw = {"tile_hint": TILES[fam]}
    if wc:
        kw["gemm1_wave_cols"] = int(wc)
    return kw


def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def region(ws: torch.Tensor, off: int, dtype, count: int) -> np.ndarray:
    nbytes = count * torch.empty(0, dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).cpu().numpy()


def run_contiguous(inp: dict, dev, precomputed=None, out=None, inplace=False, out_dtype=None,
                   packed=False, **extra):
    """One forward of a contiguous workload; returns (out, ws, info).
    out_dtype=None keeps the workload's own output type; packed=True re-lays
    the weights out with moe_pack_weights first; extra keyword arguments go
    to binding.fused_moe (expert_map, apply_weight_on_input, chunk_tokens)."""
    cfg: W.MoeConfig = inp["cfg"]
    hidden = inp["hidden"].to(dev)
    kw = dict(out_dtype=out_dtype, top_k=cfg.top_k, renormalize=cfg.renormalize, routing=cfg.scoring,
              group_count=cfg.group_count, k_group=cfg.k_group,
              group_select_mode=cfg.group_select_mode,
              routed_scaling_factor=cfg.routed_scaling_factor)
    w13, w2 = inp["w13"].to(dev), inp["w2"].to(dev)
    if cfg.fp8_block:
        packed = True                   # block-wise scales run on the packed fp8 kernels
        kw["fp8_block"] = cfg.fp8_block
    bits = WQ_BITS.get(cfg.weight, 0)
    if bits:
        packed = True                   # WNA16 codes run packed
        kw["wq_group"] = cfg.wq_group
    if packed:
        w13, w2 = B.pack_weights(w13, w2, wq_bits=bits), None
    for name in ("w13_bias", "w2_bias", "w13_scale", "w2_scale", "w13_zero", "w2_zero"):
        if inp.get(name) is not None:
            kw[name] = inp[name].to(dev)
    logits = None
    if precomputed is not None:
        kw["topk_ids"] = torch.as_tensor(precomputed[0], dtype=torch.int32).to(dev)
        kw["topk_weights"] = torch.as_tensor(precomputed[1], dtype=torch.float32).to(dev)
    else:
        logits = inp["logits"].to(dev)
    if inplace:
        out = hidden
    kw.update(extra)
    res = B.fused_moe(hidden, w13, w2, logits, out=out, **kw)
    torch.cuda.synchronize()
    return res


def oracle_route(inp: dict):
    cfg = inp["cfg"]
    return oracle.route(inp["logits"].cpu(), cfg.top_k, scoring=cfg.scoring,
                        renormalize=cfg.renormalize, group_count=cfg.group_count,
                        k_group=cfg.k_group, group_select_mode=cfg.group_select_mode,
                        routed_scaling_factor=cfg.routed_scaling_factor)


def check_routing_and_align(inp: dict, ws, info, ids_o=None, w_o=None, check_weights=True):
    """Bit-exact topk ids, counts, sorted ids, expert ids, num_post_padded;
    routing weights within TOL_WEIGHT.  Returns the oracle (ids, weights)."""
    cfg = inp["cfg"]
    M, K, E = cfg.M, cfg.top_k, cfg.E
    if ids_o is None:
        ids_o, w_o = oracle_route(inp)
        ids_g = region(ws, info.off_topk_ids, torch.int32, M * K).reshape(M, K)
        w_g = region(ws, info.off_topk_weights, torch.float32, M * K).reshape(M, K)
        bad = np.argwhere(ids_g != ids_o)
        assert bad.size == 0, f"topk ids differ at {bad[:5].tolist()}"
        if check_weights:
            err = np.abs(w_g - w_o).max()
            assert err <= TOL_WEIGHT * max(1.0, cfg.routed_scaling_factor), err
    BM = info.block_m
    counts_o, sorted_o, eids_o, npp_o = oracle.align(ids_o, E, BM)
    npp = int(region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    assert npp == npp_o
    assert np.array_equal(region(ws, info.off_expert_counts, torch.int32, E), counts_o)
    assert np.array_equal(region(ws, info.off_sorted_ids, torch.int32, npp), sorted_o)
    assert np.array_equal(region(ws, info.off_expert_ids, torch.int32, npp // BM), eids_o)
    return ids_o, w_o


def _cpu(t):
    return None if t is None else t.cpu()


def oracle_experts(inp: dict, wq_bf16: bool = False) -> oracle.Experts:
    """The workload's experts for the oracle; wq_bf16: WNA16 weights under
    the compute-type reading (see WQ_BITS).  Where the path holds z in bf16
    (bf16 activations, no fp8 requantisation), so does the oracle: the
    walkthrough keeps its activation output (intermediate_cache2) in the
    compute type."""
    cfg = inp["cfg"]
    return oracle.Experts(inp["w13"].cpu(), inp["w2"].cpu(), _cpu(inp.get("w13_scale")),
                          _cpu(inp.get("w2_scale")), _cpu(inp.get("w13_bias")),
                          _cpu(inp.get("w2_bias")), requant_z=cfg.weight == "fp8",
                          block=cfg.fp8_block, bits=WQ_BITS.get(cfg.weight, 0),
                          group=cfg.wq_group,
                          w13_zero=_cpu(inp.get("w13_zero")), w2_zero=_cpu(inp.get("w2_zero")),
                          wq_bf16=wq_bf16, z_bf16=cfg.weight != "fp8" and cfg.act == "bf16")


class Readings:
    """WNA16: the oracle's result under the compute-type reading of the
    dequantised weights, beside the exact one it accompanies (see WQ_BITS)."""

    def __init__(self, alt: np.ndarray):
        self.alt = alt


def tie_adjusted(got: np.ndarray, ref: np.ndarray, ties) -> np.ndarray:
    """Per output row, the reference closest to the device's output among the
    equally correct ones: ref plus any subset of the row's near-tie flips
    (the oracle reports at most oracle.max_ties() of them a row)."""
    ref = ref.copy()
    MT = ties.delta.shape[1]
    for n in np.nonzero(ties.count)[0]:
        c = min(int(ties.count[n]), MT)
        d = ties.delta[n, :c]
        best, best_err = ref[n], float(np.abs(got[n] - ref[n]).max())
        for mask in range(1, 1 << c):
            cand = ref[n] + d[[i for i in range(c) if mask >> i & 1]].sum(0)
            err = float(np.abs(got[n] - cand).max())
            if err < best_err:
                best, best_err = cand, err
        ref[n] = best
    return ref


def compare(cfg: W.MoeConfig, got: np.ndarray, ref: np.ndarray, what: str = "",
            ties=None) -> float:
    """Applies the dtype's tolerance; returns the error in tolerance units.
    ties (fp8): the oracle's near-tie report for the rows of ref."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    ref0 = ref
    if isinstance(ties, Readings):
        g64 = got.reshape(ref.shape).astype(np.float64)
        e_exact = float(np.abs(g64 - ref).max()) if ref.size else 0.0
        e_bf16 = float(np.abs(g64 - ties.alt).max()) if ref.size else 0.0
        print(f"[parity] {cfg.name} {what}: max err vs exact weights {e_exact:.3e}, "
              f"vs bf16 weights {e_bf16:.3e}", flush=True)
        if e_bf16 < e_exact:
            ref = ties.alt
        ties = None
    if ties is not None and ties.count.any():
        got2 = got.reshape(ref.shape).astype(np.float64)
        ref = tie_adjusted(got2, ref, ties)
        print(f"[parity] {cfg.name} {what}: {int((ties.count > 0).sum())} rows with near-tie "
              f"z codes ({int(ties.count.sum())} codes)", flush=True)
    err = float(np.abs(got.astype(np.float64) - ref).max()) if ref.size else 0.0
    if cfg.weight == "f32":
        bound = TOL_F32_ABS
    else:
        rms = float(np.sqrt(np.mean(ref0 ** 2)))
        bound = (TOL_FP8_RMS if cfg.weight == "fp8" else TOL_BF16_RMS) * rms
    print(f"[parity] {cfg.name} {what} max_abs_err={err:.3e} bound={bound:.3e} "
          f"ratio={err / bound if bound else 0:.3f}", flush=True)
    assert err <= bound, f"{what}: max abs err {err} > {bound}"
    return err / bound


def ref_tokens(inp: dict, ids_o, w_o, tokens=None, **kw):
    """The oracle's output rows of the listed tokens, and for fp8 its near-tie
    report, for WNA16 its second reading (Readings; None otherwise)."""
    cfg = inp["cfg"]
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    if cfg.weight == "fp8":
        y, _, ties = oracle.forward_tokens(oracle_experts(inp), acts, ids_o, w_o, tokens=tokens,
                                           tie_window=TIE_WINDOW, **kw)
        return y, ties
    y, _ = oracle.forward_tokens(oracle_experts(inp), acts, ids_o, w_o, tokens=tokens, **kw)
    if cfg.weight in WQ_BITS:
        y2, _ = oracle.forward_tokens(oracle_experts(inp, wq_bf16=True), acts, ids_o, w_o,
                                      tokens=tokens, **kw)
        return y, Readings(y2)
    return y, None


def ref_rows(inp: dict, acts, rows, experts):
    """The oracle's expert outputs of (activation row, expert) pairs, and for
    fp8 its near-tie report, for WNA16 its second reading (Readings; None
    otherwise)."""
    if inp["cfg"].weight == "fp8":
        o, _, ties = oracle.expert_rows(oracle_experts(inp), acts, rows, experts,
                                        tie_window=TIE_WINDOW)
        return o, ties
    o, _ = oracle.expert_rows(oracle_experts(inp), acts, rows, experts)
    if inp["cfg"].weight in WQ_BITS:
        o2, _ = oracle.expert_rows(oracle_experts(inp, wq_bf16=True), acts, rows, experts)
        return o, Readings(o2)
    return o, None


def reduce_rows(inp: dict, rows, o_ref, ties=None):
    """The batched format's weighted reduction of expert rows through the
    token map, y[t] = sum_j w[t, j] o[row(t, j)] (entries -1: no row here),
    and the near-tie report carried through it."""
    cfg = inp["cfg"]
    if isinstance(ties, Readings):
        y, _ = reduce_rows(inp, rows, o_ref)
        y2, _ = reduce_rows(inp, rows, ties.alt)
        return y, Readings(y2)
    pos = {r: i for i, r in enumerate(rows)}
    tmap = inp["token_map"].cpu().numpy().astype(np.int64)
    wts = inp["token_map_w"].cpu().numpy().astype(np.float64)
    y = np.zeros((cfg.M, cfg.H))
    rt = None
    if ties is not None:
        MT = ties.delta.shape[1]
        rt = oracle.Ties(np.zeros(cfg.M, np.int32), np.zeros((cfg.M, MT, cfg.H)))
    for t in range(cfg.M):
        for j in range(cfg.top_k):
            r = tmap[t, j]
            if r < 0:
                continue
            y[t] += wts[t, j] * o_ref[pos[r]]
            if rt is not None:
                n = pos[r]
                for i in range(min(int(ties.count[n]), ties.delta.shape[1])):
                    if rt.count[t] < rt.delta.shape[1]:
                        rt.delta[t, rt.count[t]] = wts[t, j] * ties.delta[n, i]
                    rt.count[t] += 1
    return y, rt


def check_output(inp: dict, out: torch.Tensor, ids_o, w_o, tokens=None, what=""):
    cfg = inp["cfg"]
    y, ties = ref_tokens(inp, ids_o, w_o, tokens=tokens)
    got = out.float().cpu().numpy()
    if tokens is not None:
        got = got[np.asarray(tokens)]
    return compare(cfg, got, y, what, ties=ties)


def run_batched(inp: dict, dev, reduce=False, out_dtype=None, packed=False, **extra):
    cfg = inp["cfg"]
    kw = {"out_dtype": out_dtype, **extra}
    w13, w2 = inp["w13"].to(dev), inp["w2"].to(dev)
    if cfg.fp8_block:
        packed = True
        kw["fp8_block"] = cfg.fp8_block
    bits = WQ_BITS.get(cfg.weight, 0)
    if bits:
        packed = True
        kw["wq_group"] = cfg.wq_group
    if packed:
        w13, w2 = B.pack_weights(w13, w2, wq_bits=bits), None
    for name in ("w13_scale", "w2_scale", "w13_bias", "w2_bias", "w13_zero", "w2_zero"):
        if inp.get(name) is not None:
            kw[name] = inp[name].to(dev)
    if reduce:
        kw["token_map"] = inp["token_map"].to(dev)
        kw["token_map_w"] = inp["token_map_w"].to(dev)
    res = B.fused_moe_batched(inp["hidden"].to(dev), inp["expert_num_tokens"].to(dev),
                              w13, w2, M=cfg.M, top_k=cfg.top_k,
                              **kw)
    torch.cuda.synchronize()
    return res


def check_batched_tilelist(inp, ws, info):
    cfg = inp["cfg"]
    T, BM = inp["max_tokens"], info.block_m
    counts = inp["expert_num_tokens"].cpu().numpy()
    npp = int(region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    padded = -(-counts // BM) * BM
    assert npp == padded.sum()
    sorted_g = region(ws, info.off_sorted_ids, torch.int32, npp)
    ref = np.concatenate([np.concatenate([e * T + np.arange(c), np.full(p - c, cfg.E * T)])
                          for e, (c, p) in enumerate(zip(counts, padded))]).astype(np.int32)
    assert np.array_equal(sorted_g, ref)
    eids = region(ws, info.off_expert_ids, torch.int32, npp // BM)
    assert np.array_equal(eids, np.repeat(np.arange(cfg.E), padded // BM))


def batched_rows(inp, sample=None):
    """(flat slab rows, expert of each row) of the valid rows, optionally a sample."""
    T = inp["max_tokens"]
    counts = inp["expert_num_tokens"].cpu().numpy()
    rows = np.concatenate([e * T + np.arange(c) for e, c in enumerate(counts)])
    if sample is not None and sample < rows.size:
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(rows, size=sample, replace=False))
    return rows.astype(np.int64), (rows // T).astype(np.int32)


def check_rounded(out16: torch.Tensor, out32: torch.Tensor):
    """The bf16 output is the float32 result rounded to nearest-even, bit for bit."""
    assert out16.dtype == torch.bfloat16 and out32.dtype == torch.float32
    ref = out32.to(torch.bfloat16)
    same = out16.view(torch.int16) == ref.view(torch.int16)
    assert bool(same.all()), f"{int((~same).sum())} bf16 outputs are not RNE(float32 result)"


# ---------------------------------------------------------------- tile coverage
# Row heights of the GEMM tile families that can run a weight type: a chunk of
# an expert's rows is one tile's rows.  Sampling the first and last row of
# every chunk of every height reaches every (expert, row chunk) tile whatever
# family the library picks, with all its columns.
CHUNK_HEIGHTS = {"fp8": (128,), "default": (32, 64, 160, 256)}


def chunk_positions(counts: np.ndarray, offsets: np.ndarray, heights) -> tuple:
    """Padded positions of the first and last real row of every row chunk
    (expert e's count rows dealt out evenly over ceil(count / CH) chunks in
    16-row strips, as the GEMM schedule does).  Returns (positions, chunks
    per height)."""
    pos, nchunks = set(), {}
    for CH in heights:
        n = 0
        for e in np.nonzero(counts)[0]:
            c, base = int(counts[e]), int(offsets[e])
            U = -(-c // 16)
            nch = -(-c // CH)
            q, extra = divmod(U, nch)
            for j in range(nch):
                u0 = j * q + min(j, extra)
                rows = min(16 * (q + (j < extra)), c - 16 * u0)
                pos.add(base + 16 * u0)
                pos.add(base + 16 * u0 + rows - 1)
            n += nch
        nchunks[CH] = n
    return np.array(sorted(pos), dtype=np.int64), nchunks


def expert_output_rows(ws, info, positions, H, dev) -> np.ndarray:
    """Each sampled routed item's expert output o[p] (+ o2[p] when the second
    GEMM ran split in K), float32 from the workspace."""
    rows = info.max_sorted_len
    o = ws[info.off_o:info.off_o + rows * H * 4].view(torch.float32).view(rows, H)
    idx = torch.as_tensor(positions, device=dev)
    got = o[idx]
    if info.off_o2:
        o2 = ws[info.off_o2:info.off_o2 + rows * H * 4].view(torch.float32).view(rows, H)
        got = got + o2[idx]
    return got.cpu().numpy()


def _z_elem_bytes(cfg) -> int:
    return 1 if cfg.weight == "fp8" else (4 if cfg.act == "f32" else 2)


def z_rows(ws, info, cfg, positions, dev) -> np.ndarray:
    """The workspace's z rows at padded positions: fp8 codes (uint8), else
    float values."""
    I, es = cfg.I, _z_elem_bytes(cfg)
    raw = ws[info.off_z:info.off_z + info.max_sorted_len * I * es]
    dt = {1: torch.uint8, 2: torch.bfloat16, 4: torch.float32}[es]
    z = raw.view(dt).view(info.max_sorted_len, I)[torch.as_tensor(positions, device=dev)]
    return z.cpu().numpy() if es == 1 else z.float().cpu().numpy()


def _fp8_decode(c):
    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()


def _fp8_step(v):
    """The E4M3FN spacing at magnitude v (2^-9 below the normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    return 2.0 ** (e - 3)


def check_z_codes(inp, ws, info, acts, rows, experts, positions, dev, what):
    """fp8 path: the z codes and group scales at `positions` against the
    oracle's for (activation row, expert) pairs (rows, experts)."""
    cfg = inp["cfg"]
    I = cfg.I
    G = I // 128
    zs_ld = info.max_sorted_len + 256                    # group-major [I/128][zs_ld]
    sall = region(ws, info.off_z_scale, torch.float32, G * zs_ld).reshape(G, zs_ld)
    codes, scales, alt = oracle.expert_z_codes(oracle_experts(inp), acts, rows, experts,
                                               tie_window=TIE_WINDOW)
    got = z_rows(ws, info, cfg, positions, dev)
    got_s = sall[:, positions].T
    srel = np.abs(got_s.astype(np.float64) / scales - 1.0).max()
    assert srel <= Z_SCALE_RTOL, f"{what}: z scales differ by {srel:.2e} relative"
    t_or, t_dev = _fp8_decode(codes), _fp8_decode(got)
    diff = got != codes
    far = np.abs(t_dev - t_or) > _fp8_step(np.maximum(np.abs(t_or), np.abs(t_dev))) + Z_ABS_TOL
    ties = int((diff & (alt >= 0) & (got.astype(np.int16) == alt)).sum())
    print(f"[z] {what}: {got.size} codes, {int(diff.sum())} differ ({ties} of them at "
          f"reported near-ties, {int((alt >= 0).sum())} reported), scale rel {srel:.1e}",
          flush=True)
    bad = np.argwhere(far)
    assert bad.size == 0, (f"{what}: {len(bad)} z codes more than a step off, first (item, "
                           f"column) {bad[:5].tolist()}")
    assert diff.mean() <= Z_MAX_FRAC, f"{what}: {diff.mean():.3%} of the codes differ"
    worst = diff.mean(axis=1).max()
    assert worst <= Z_MAX_ITEM_FRAC, f"{what}: {worst:.3%} of one item's codes differ"


def check_z(inp, ws, info, acts, rows, experts, positions, dev, what):
    """z at `positions` against the oracle's z of (activation row, expert)
    pairs; fp8 codes through check_z_codes; WNA16 against the closer of its
    two readings (see WQ_BITS)."""
    cfg = inp["cfg"]
    if cfg.weight == "fp8":
        check_z_codes(inp, ws, info, acts, rows, experts, positions, dev, what)
        return
    got = z_rows(ws, info, cfg, positions, dev)
    best = None
    for wq_bf16 in ((False, True) if cfg.weight in WQ_BITS else (False,)):
        ref = oracle.expert_z(oracle_experts(inp, wq_bf16=wq_bf16), acts, rows, experts)
        rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
        tol = Z_REL[_z_elem_bytes(cfg)] * np.abs(ref) + Z_RMS * rms
        ratio = np.abs(got - ref) / tol
        if best is None or ratio.max() < best[0].max():
            best = (ratio, wq_bf16)
    ratio = best[0]
    reading = " (bf16 weights)" if best[1] else ""
    print(f"[z] {what}: {got.size} values, max error {ratio.max():.3f} of the bound{reading}",
          flush=True)
    bad = np.argwhere(ratio > 1.0)
    assert bad.size == 0, f"{what}: {len(bad)} z values off, first (item, column) {bad[:5].tolist()}"


def check_z_all_contiguous(inp, ws, info, ids_o, dev, what):
    """check_z over every routed item of a contiguous forward (its padded
    position, token and expert from the workspace's sorted ids)."""
    cfg = inp["cfg"]
    npp = int(region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    sorted_ids = region(ws, info.off_sorted_ids, torch.int32, npp)
    pos = np.nonzero(sorted_ids < cfg.M * cfg.top_k)[0]
    r = sorted_ids[pos]
    tokens, experts = (r // cfg.top_k).astype(np.int64), ids_o.reshape(-1)[r]
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    check_z(inp, ws, info, acts, tokens, experts.astype(np.int32), pos, dev, what)


def check_tiles_contiguous(inp, ws, info, dev, E_local=None):
    """Every (expert, row chunk) tile of a contiguous forward: the expert
    outputs of its first and last rows against the oracle's expert FFN of
    that token.  Returns the tokens of the sampled items."""
    cfg = inp["cfg"]
    E = E_local or cfg.E
    counts = region(ws, info.off_expert_counts, torch.int32, E)
    offs = region(ws, info.off_expert_offsets, torch.int32, E + 1)
    heights = CHUNK_HEIGHTS.get(cfg.weight, CHUNK_HEIGHTS["default"])
    pos, nch = chunk_positions(counts, offs, heights)
    npp = int(region(ws, info.off_num_post_padded, torch.int32, 1)[0])
    sorted_ids = region(ws, info.off_sorted_ids, torch.int32, npp)
    sid = sorted_ids[pos]
    assert (sid < cfg.M * cfg.top_k).all(), "a sampled position is padding"
    experts = np.searchsorted(offs, pos, side="right") - 1
    tokens = (sid // cfg.top_k).astype(np.int64)
    print(f"[tiles] {cfg.name}: {len(pos)} item rows over chunks {nch} of "
          f"{int((counts > 0).sum())} experts", flush=True)
    acts = oracle.Acts(inp["hidden"].cpu(), quantize=cfg.weight == "fp8", block=cfg.fp8_block)
    check_z(inp, ws, info, acts, tokens, experts.astype(np.int32), pos, dev,
            "z rows of every tile")
    ref, ties = ref_rows(inp, acts, tokens, experts.astype(np.int32))
    got = expert_output_rows(ws, info, pos, cfg.H, dev)
    compare(cfg, got, ref, "expert rows of every tile", ties=ties)
    return np.unique(tokens)


def check_tiles_batched(inp, ws, info, out, dev):
    """Every (expert, row chunk) tile of a batched forward without reduce:
    the first and last rows' outputs against the oracle's expert FFN."""
    cfg = inp["cfg"]
    T = inp["max_tokens"]
    counts = region(ws, info.off_expert_counts, torch.int32, cfg.E)
    offs = region(ws, info.off_expert_offsets, torch.int32, cfg.E + 1)
    heights = CHUNK_HEIGHTS.get(cfg.weight, CHUNK_HEIGHTS["default"])
    pos, nch = chunk_positions(counts, offs, heights)
    experts = np.searchsorted(offs, pos, side="right") - 1
    rows = experts * T + (pos - offs[experts])
    print(f"[tiles] {cfg.name}: {len(pos)} slab rows over chunks {nch} of "
          f"{int((counts > 0).sum())} experts", flush=True)
    acts = oracle.Acts(inp["hidden"].cpu(), scale=_cpu(inp.get("a_scale")),
                       quantize=cfg.weight == "fp8" and inp["hidden"].dtype != torch.float8_e4m3fn,
                       block=cfg.fp8_block)
    check_z(inp, ws, info, acts, rows, experts.astype(np.int32), pos, dev,
            "z rows of every tile")
    ref, ties = ref_rows(inp, acts, rows, experts.astype(np.int32))
    got = out.reshape(-1, cfg.H)[torch.as_tensor(rows, device=dev)].float().cpu().numpy()
    compare(cfg, got, ref, "slab rows of every tile", ties=ties)
    return rows
