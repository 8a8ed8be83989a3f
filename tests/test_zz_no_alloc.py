"""moe_forward_static, the allocation-free entry point, against moe_forward.

Both run the same kernels; the static one takes its workspace from the
library's device array, which keeps the previous call's contents.  Each case
runs two forwards in a row through the static entry, the second on a
smaller input than the first (so stale data of the first call sits in the
array), and requires each output to equal moe_forward's bit for bit and to
meet the oracle's bar."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

PAIRS = [
    ("decode", W.DECODE_SMALL_EXPERTS, W.DECODE_SMALL_EXPERTS.scaled(name="decode_m8", M=8)),
    ("prefill_grouped_bias",
     W.DEEPSEEK_GROUPED.scaled(name="sa_grouped", M=600, H=256, I=512, E=64),
     W.DEEPSEEK_GROUPED.scaled(name="sa_grouped_small", M=48, H=256, I=512, E=64)),
    ("fp8_contiguous", W.MIXTRAL_PREFILL.scaled(name="sa_fp8", M=300, H=512, I=256, weight="fp8"),
     W.MIXTRAL_PREFILL.scaled(name="sa_fp8_small", M=20, H=512, I=256, weight="fp8")),
]


def _check(inp, dev, what, **kw):
    ref, ws, info = GH.run_contiguous(inp, dev, out_dtype=torch.float32, **kw)
    got, ws2, info2 = GH.run_contiguous(inp, dev, out_dtype=torch.float32, static=True, **kw)
    assert ws2 is None and info2 is None
    assert torch.equal(got, ref), f"{what}: static output differs from moe_forward's"
    ids_o, w_o = GH.oracle_route(inp)
    cfg = inp["cfg"]
    tokens = None if cfg.M <= 64 else np.unique(np.r_[0, cfg.M - 1,
                                                      np.arange(0, cfg.M, cfg.M // 40)])
    GH.check_output(inp, got, ids_o, w_o, tokens=tokens, what=what)


@pytest.mark.parametrize("name,big,small", PAIRS, ids=[p[0] for p in PAIRS])
def test_static_entry_two_calls_second_smaller(name, big, small):
    dev = GH.device()
    for cfg in (big, small):
        print(f"[case] static {name} {cfg.name} M={cfg.M}", flush=True)
        inp = W.make_inputs(cfg, 501, device=dev)
        _check(inp, dev, f"{name}/{cfg.name}")


def test_static_entry_batched_two_calls():
    dev = GH.device()
    for M in (512, 64):
        cfg = W.BATCHED_FP8.scaled(name=f"sa_batched_{M}", M=M, H=256, I=256, E=8)
        print(f"[case] static batched M={M}", flush=True)
        inp = W.make_inputs(cfg, 502)
        for reduce in (False, True):
            ref, _, _ = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32)
            got, ws, _ = GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32,
                                        static=True)
            assert ws is None
            if reduce:
                assert torch.equal(got, ref)
            else:
                rows = torch.as_tensor(GH.batched_rows(inp)[0], device=dev)
                assert torch.equal(got.reshape(-1, cfg.H)[rows], ref.reshape(-1, cfg.H)[rows])


def test_static_entry_limit_and_chunking():
    """A batch whose workspace exceeds the array is refused with nothing
    enqueued; the same batch in chunks runs and equals moe_forward."""
    dev = GH.device()
    cfg = W.MIXTRAL_PREFILL.scaled(name="sa_long", M=20000, H=1024, I=1024, E=8)
    p = B.Problem(M=cfg.M, H=cfg.H, I=cfg.I, E=cfg.E, top_k=cfg.top_k, renormalize=True)
    assert B.moe_workspace_shapes(p.c()).bytes > B.MOE_STATIC_WORKSPACE_BYTES
    inp = W.make_inputs(cfg, 503, device=dev)
    out = torch.full((cfg.M, cfg.H), 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(B.MoeError) as err:
        GH.run_contiguous(inp, dev, out=out, static=True)
    assert err.value.status == B.MOE_ERR_STATIC_LIMIT
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
    p.chunk_tokens = 4096
    assert B.moe_workspace_shapes(p.c()).bytes <= B.MOE_STATIC_WORKSPACE_BYTES
    print("[case] static chunked M=20000", flush=True)
    _check(inp, dev, "static chunked", chunk_tokens=4096)
    # and a smaller call after it
    inp = W.make_inputs(cfg.scaled(name="sa_long_small", M=300), 504, device=dev)
    _check(inp, dev, "static after chunked")
