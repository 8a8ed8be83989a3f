"""Batched slabs as an expert-parallel dispatch hands them over, and the
device status word.

vLLM's "Fused MoE Modular Kernel" page sizes the batched activations as
[E_local, max_tokens, H] with max_tokens = num_dispatchers x
max_num_tokens_per_rank (FusedMoEPrepareAndFinalize), so a slab has room for
every dispatcher's full batch while the dispatchers together send fewer
tokens: max_tokens > M, ragged per-dispatcher batches, NaN past each count.
This rank holds a share of the global experts; token copies routed to
experts held elsewhere have no slab row (token_map -1) and the reduce sums
this rank's partial output.

The status tests hand the path device-side data the host cannot check (ids,
counts, token-map entries, a broken row promise) and require that the bad
entries contribute nothing, the rest is computed, and the status word names
what happened."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
import oracle
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu


def dispatch_slabs(x, ids, local0, E_local, per_rank, batches, H):
    """Slabs of the local experts [local0, local0 + E_local) filled in
    dispatcher order (dispatcher d's tokens, ascending, then d + 1's), NaN
    past each count; token_map[t, j] = e * T + row, or -1 for a copy held
    elsewhere."""
    R = len(batches)
    T = R * per_rank
    M, K = ids.shape
    xb = torch.full((E_local, T, H), float("nan"), dtype=x.dtype)
    counts = np.zeros(E_local, np.int32)
    tmap = np.full((M, K), -1, np.int32)
    starts = np.concatenate([[0], np.cumsum(batches)])
    for d in range(R):
        for t in range(starts[d], starts[d + 1]):
            for j in range(K):
                e = int(ids[t, j]) - local0
                if 0 <= e < E_local:
                    xb[e, counts[e]] = x[t]
                    tmap[t, j] = e * T + counts[e]
                    counts[e] += 1
    return xb, torch.from_numpy(counts), torch.from_numpy(tmap), T


@pytest.mark.parametrize("weight", ["bf16", "fp8"])
def test_batched_slabs_from_four_dispatchers(weight):
    dev = GH.device()
    Eg, E_local, local0, K, H, I = 16, 4, 4, 4, 256, 384
    per_rank, batches = 48, [40, 13, 0, 27]
    M = sum(batches)
    gen = torch.Generator().manual_seed(301)
    x = torch.randn(M, H, generator=gen).to(torch.bfloat16)
    logits = torch.randn(M, Eg, generator=gen)
    ids, wts = oracle.route(logits, K, scoring="softmax", renormalize=True)
    xb, counts, tmap, T = dispatch_slabs(x, ids, local0, E_local, per_rank, batches, H)
    assert T == 192 > M
    w13 = torch.randn(E_local, H, 2 * I, generator=gen) / H ** 0.5
    w2 = torch.randn(E_local, I, H, generator=gen) / I ** 0.5
    cfg = W.MoeConfig(f"dispatch4_{weight}", M=M, H=H, I=I, E=E_local, top_k=K,
                      fmt="batched", weight=weight)
    inp = {"cfg": cfg, "hidden": xb, "expert_num_tokens": counts, "max_tokens": T,
           "token_map": tmap, "token_map_w": torch.from_numpy(wts.astype(np.float32)),
           "w13_bias": None, "w2_bias": None}
    if weight == "fp8":
        inp["w13"], inp["w13_scale"] = W.quantize_weight_fp8(w13)
        inp["w2"], inp["w2_scale"] = W.quantize_weight_fp8(w2)
    else:
        inp["w13"], inp["w2"] = w13.to(torch.bfloat16), w2.to(torch.bfloat16)
    print(f"[case] {cfg.name} M={M} T={T} rows={int(counts.sum())}", flush=True)
    # this rank's partial output: the oracle over the global routing with the
    # experts held elsewhere mapped to -1
    emap = np.full(Eg, -1, np.int32)
    emap[local0:local0 + E_local] = np.arange(E_local)
    acts = oracle.Acts(x, quantize=weight == "fp8")
    fp8 = weight == "fp8"
    y, _, yt = oracle.forward_tokens(GH.oracle_experts(inp), acts, ids, wts, expert_map=emap,
                                     tie_window=GH.TIE_WINDOW if fp8 else 1e-30)
    for packed in (False, True):
        out, ws, info = GH.run_batched(inp, dev, reduce=True, out_dtype=torch.float32,
                                       packed=packed)
        GH.check_batched_tilelist(inp, ws, info)
        assert B.device_status(ws, info) == 0
        GH.compare(cfg, out.cpu().numpy(), y, f"dispatch reduce packed={packed}",
                   ties=yt if fp8 else None)
        slabs, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32, packed=packed)
        rows, experts = GH.batched_rows(inp)
        ref, ties = GH.ref_rows(inp, oracle.Acts(xb, quantize=fp8), rows, experts)
        got = slabs.reshape(-1, H)[torch.as_tensor(rows, device=dev)].cpu().numpy()
        GH.compare(cfg, got, ref, f"dispatch slab rows packed={packed}", ties=ties)


def _small_batched(seed, counts, T, H=128, I=128, K=2):
    E = len(counts)
    gen = torch.Generator().manual_seed(seed)
    cfg = W.MoeConfig("status_batched", M=0, H=H, I=I, E=E, top_k=K, fmt="batched")
    xb = torch.full((E, T, H), float("nan"))
    for e, c in enumerate(counts):
        c = min(max(c, 0), T)
        xb[e, :c] = torch.randn(c, H, generator=gen)
    return cfg, {"cfg": cfg, "hidden": xb.to(torch.bfloat16),
                 "expert_num_tokens": torch.tensor(counts, dtype=torch.int32),
                 "w13": (torch.randn(E, H, 2 * I, generator=gen) / H ** 0.5).to(torch.bfloat16),
                 "w2": (torch.randn(E, I, H, generator=gen) / I ** 0.5).to(torch.bfloat16),
                 "max_tokens": T, "w13_bias": None, "w2_bias": None}


def test_status_rows_overflow_reduce_gives_zeros():
    """Slabs holding more valid rows than the promised M * top_k: nothing is
    computed, the reduced output is zero, the status word says so."""
    dev = GH.device()
    cfg, inp = _small_batched(310, [30, 20, 25], T=32)
    M, K = 20, 2                                  # promise 40 rows; the slabs hold 75
    tmap = torch.tensor([[e * 32 + i % 20, ((e + 1) % 3) * 32 + i % 20]
                         for i, e in zip(range(M), [0, 1, 2] * 7)], dtype=torch.int32)
    out = torch.full((M, cfg.H), 7.0, device=dev)
    out, ws, info = B.fused_moe_batched(
        inp["hidden"].to(dev), inp["expert_num_tokens"].to(dev), inp["w13"].to(dev),
        inp["w2"].to(dev), token_map=tmap.to(dev), token_map_w=torch.ones(M, K, device=dev),
        out=out, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert B.device_status(ws, info) == B.MOE_DEV_ROWS_OVERFLOW
    assert int(out.abs().max()) == 0


def test_status_rows_overflow_slabs_untouched():
    dev = GH.device()
    cfg, inp = _small_batched(311, [30, 20, 25], T=32)
    out = torch.full((3, 32, cfg.H), 7.0, dtype=torch.bfloat16, device=dev)
    out, ws, info = B.fused_moe_batched(
        inp["hidden"].to(dev), inp["expert_num_tokens"].to(dev), inp["w13"].to(dev),
        inp["w2"].to(dev), M=20, top_k=2, out=out)
    torch.cuda.synchronize()
    assert B.device_status(ws, info) == B.MOE_DEV_ROWS_OVERFLOW
    assert bool((out == 7.0).all())
    # the same slabs without the row promise are computed in full
    out, ws, info = B.fused_moe_batched(
        inp["hidden"].to(dev), inp["expert_num_tokens"].to(dev), inp["w13"].to(dev),
        inp["w2"].to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert B.device_status(ws, info) == 0
    rows, experts = GH.batched_rows(inp)
    ref, _ = oracle.expert_rows(GH.oracle_experts(inp), oracle.Acts(inp["hidden"]), rows,
                                experts)
    GH.compare(cfg, out.reshape(-1, cfg.H)[torch.as_tensor(rows, device=dev)].cpu().numpy(),
               ref, "no promise")


def test_status_count_clamped():
    """expert_num_tokens outside [0, max_tokens] is clamped: the rows inside
    the slab are computed, and the status word reports the clamp."""
    dev = GH.device()
    cfg, inp = _small_batched(312, [40, -3, 7], T=32)
    out, ws, info = GH.run_batched(inp, dev, out_dtype=torch.float32)
    assert B.device_status(ws, info) == B.MOE_DEV_COUNT_CLAMPED
    counts = GH.region(ws, info.off_expert_counts, torch.int32, 3)
    assert list(counts) == [32, 0, 7]
    rows = np.concatenate([np.arange(32), 64 + np.arange(7)])
    experts = (rows // 32).astype(np.int32)
    ref, _ = oracle.expert_rows(GH.oracle_experts(inp), oracle.Acts(inp["hidden"]), rows,
                                experts)
    GH.compare(cfg, out.reshape(-1, cfg.H)[torch.as_tensor(rows, device=dev)].cpu().numpy(),
               ref, "clamped")


def test_status_token_map_entries():
    """token_map entries that name no valid slab row (past a count, past
    the slabs, negative other than -1) contribute nothing and set
    MOE_DEV_TOKEN_MAP; -1 entries contribute nothing silently."""
    dev = GH.device()
    cfg, inp = _small_batched(313, [12, 11, 9], T=16)
    M, K = 16, 2                                   # 32 copies, one per valid slab row
    rng = np.random.default_rng(9)
    valid = np.concatenate([e * 16 + np.arange(c) for e, c in enumerate([12, 11, 9])])
    tmap = rng.choice(valid, size=(M, K), replace=False).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, (M, K)).astype(np.float32)
    rows_all, experts_all = GH.batched_rows(inp)
    ref_rows, _ = oracle.expert_rows(GH.oracle_experts(inp), oracle.Acts(inp["hidden"]),
                                     rows_all, experts_all)
    pos = {int(r): i for i, r in enumerate(rows_all)}

    def expect(tm):
        y = np.zeros((M, cfg.H))
        for t in range(M):
            for j in range(K):
                if int(tm[t, j]) in pos:
                    y[t] += float(tw[t, j]) * ref_rows[pos[int(tm[t, j])]]
        return y

    def run(tm):
        out, ws, info = B.fused_moe_batched(
            inp["hidden"].to(dev), inp["expert_num_tokens"].to(dev), inp["w13"].to(dev),
            inp["w2"].to(dev), token_map=torch.from_numpy(tm).to(dev),
            token_map_w=torch.from_numpy(tw).to(dev), out_dtype=torch.float32)
        torch.cuda.synchronize()
        return out, B.device_status(ws, info)

    out, st = run(tmap)
    assert st == 0
    GH.compare(cfg, out.cpu().numpy(), expect(tmap), "valid map")
    held = tmap.copy()
    held[::3, 1] = -1                              # copies served by another rank
    out, st = run(held)
    assert st == 0
    GH.compare(cfg, out.cpu().numpy(), expect(held), "map with -1")
    bad = tmap.copy()
    bad[0, 0] = 0 * 16 + 12                        # past expert 0's count
    bad[1, 1] = 3 * 16                             # past the slabs
    bad[2, 0] = -7
    out, st = run(bad)
    assert st == B.MOE_DEV_TOKEN_MAP
    GH.compare(cfg, out.cpu().numpy(), expect(bad), "map with bad entries")


@pytest.mark.parametrize("M", [40, 4500], ids=["one_workgroup_align", "multi_workgroup_align"])
def test_status_precomputed_ids_and_map_out_of_range(M):
    """Precomputed ids outside [0, experts) and expert-map values outside
    [-1, E) give their items no row and set MOE_DEV_ID_RANGE; above 16384
    routed items the align runs over several workgroups."""
    dev = GH.device()
    E, K = 8, 4
    cfg = W.MIXTRAL_PREFILL.scaled(name="status_ids", M=M, H=64, I=64, E=E, top_k=K)
    inp = W.make_inputs(cfg, 314)
    rng = np.random.default_rng(3)
    ids = np.argsort(rng.random((M, E)), axis=1)[:, :K].astype(np.int32)
    w = rng.uniform(0.1, 1.0, (M, K)).astype(np.float32)
    tokens = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 24, replace=False)]))
    out, ws, info = GH.run_contiguous(inp, dev, precomputed=(ids, w), out_dtype=torch.float32)
    assert B.device_status(ws, info) == 0
    bad = ids.copy()
    bad[0, 1], bad[M - 1, 3], bad[M // 2, 0] = E, -2, 1 << 20
    out, ws, info = GH.run_contiguous(inp, dev, precomputed=(bad, w), out_dtype=torch.float32)
    assert B.device_status(ws, info) == B.MOE_DEV_ID_RANGE
    # the same items with weight 0 on a valid expert: the oracle's reading
    fixed, wz = bad.copy(), w.astype(np.float64)
    badm = (bad < 0) | (bad >= E)
    fixed[badm], wz[badm] = 0, 0.0
    GH.check_output(inp, out, fixed, wz, tokens=tokens, what="ids out of range")
    # an expert map naming a local expert that does not exist
    emap = torch.tensor([0, 1, 2, 3, -1, 9, 5, -1], dtype=torch.int32)
    inp4 = W.make_inputs(cfg.scaled(name="status_map"), 315)
    inp4["w13"], inp4["w2"] = inp4["w13"][:6].contiguous(), inp4["w2"][:6].contiguous()
    out, ws, info = GH.run_contiguous(inp4, dev, precomputed=(ids, w), out_dtype=torch.float32,
                                      expert_map=emap.to(dev))
    assert B.device_status(ws, info) == B.MOE_DEV_ID_RANGE
    y, _ = oracle.forward_tokens(GH.oracle_experts(inp4), oracle.Acts(inp4["hidden"]), ids,
                                 w.astype(np.float64), tokens=tokens,
                                 expert_map=np.array([0, 1, 2, 3, -1, -1, 5, -1], np.int32))
    GH.compare(cfg, out.cpu().numpy()[tokens], y, "map out of range")
