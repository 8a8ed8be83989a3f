"""The bounds-checked build (libmoe_checked.so) against the release build.

In the checked build every index the kernels take from device data (the GEMM
tile table, the sorted ids behind row gathers and output rows, the reduce's
row map) is checked against its buffer before it is used.  On valid inputs
no check may fire and nothing else changes: each case here runs both builds
on the same inputs and requires bit-equal outputs and a clear status word
from the checked one.  The cases cover every GEMM family the checks touch
(DMA tiles of 256 / 160 / 32 rows, the register-staged tiles, the fp8 DMA
tiles, WNA16), multi-chunk experts, the second GEMM split in K, an expert
shard and the batched format with and without its reduce."""
import numpy as np
import pytest
import torch

import gpu_harness as GH
from mixture_experts_ffn_router_amd import binding as B
from mixture_experts_ffn_router_amd import workloads as W

pytestmark = pytest.mark.gpu

CONTIGUOUS = [
    ("grouped_dma160", W.DEEPSEEK_GROUPED.scaled(name="chk_grouped", M=512, H=256, I=256, E=8,
                                                 top_k=4, group_count=4, k_group=2),
     dict(packed=True)),
    ("dma256_plain", W.MIXTRAL_PREFILL.scaled(name="chk_256", M=640, H=256, I=320, E=4),
     GH.tile_kwargs("dma256")),
    ("reg64_bias", W.MIXTRAL_PREFILL.scaled(name="chk_reg", M=64, H=256, I=384, E=8, bias=True),
     GH.tile_kwargs("reg64")),
    ("k_split", W.MIXTRAL_PREFILL.scaled(name="chk_ksplit", M=96, H=256, I=1040, E=4, bias=True),
     dict(packed=True, **GH.tile_kwargs("dma160"))),
    ("decode", W.DECODE_SMALL_EXPERTS.scaled(name="chk_decode", M=8, H=256, I=256, E=32,
                                             top_k=4), dict(packed=True)),
    ("fp8_per_channel", W.MIXTRAL_PREFILL.scaled(name="chk_fp8", M=256, H=256, I=256, E=8,
                                                 weight="fp8"), dict(packed=True)),
    ("w4a16_zero", W.DECODE_SMALL_EXPERTS.scaled(name="chk_w4", M=8, H=320, I=256, E=32,
                                                 top_k=4, weight="u4", wq_zero=True), {}),
    ("w8a16_g32_dma160", W.MIXTRAL_PREFILL.scaled(name="chk_w8", M=400, H=256, I=256, E=4,
                                                  weight="u8", wq_group=32, bias=True),
     GH.tile_kwargs("dma160")),
    ("fp8_block", W.MIXTRAL_PREFILL.scaled(name="chk_fp8_block", M=300, H=208, I=256, E=4,
                                           weight="fp8", fp8_block=128, bias=True), {}),
]


def _both(run):
    rel = run()
    with B.checked_library() as lib:
        assert lib.moe_version().decode().endswith("checked")
        chk = run()
    return rel, chk


@pytest.mark.parametrize("name,cfg,kw", CONTIGUOUS, ids=[c[0] for c in CONTIGUOUS])
def test_checked_equals_release(name, cfg, kw):
    dev = GH.device()
    inp = W.make_inputs(cfg, 5100 + [c[0] for c in CONTIGUOUS].index(name))
    print(f"[case] checked {name}", flush=True)
    (out_r, ws_r, info_r), (out_c, ws_c, info_c) = _both(
        lambda: GH.run_contiguous(inp, dev, out_dtype=torch.float32, **kw))
    assert B.device_status(ws_r, info_r) == 0
    assert B.device_status(ws_c, info_c) == 0
    assert torch.equal(out_r, out_c)


def test_checked_expert_shard():
    dev = GH.device()
    cfg = W.DEEPSEEK_GROUPED.scaled(name="chk_shard", M=384, H=256, I=256, E=16, top_k=4,
                                    group_count=4, k_group=2)
    inp = W.make_inputs(cfg, 5150)
    emap = torch.full((cfg.E,), -1, dtype=torch.int32)
    emap[4:12] = torch.arange(8, dtype=torch.int32)
    print("[case] checked expert shard", flush=True)
    (out_r, ws_r, info_r), (out_c, ws_c, info_c) = _both(
        lambda: GH.run_contiguous(inp, dev, out_dtype=torch.float32, packed=True,
                                  expert_map=emap.to(dev)))
    assert B.device_status(ws_c, info_c) == 0
    assert torch.equal(out_r, out_c)


@pytest.mark.parametrize("reduce", [False, True], ids=["slabs", "reduce"])
def test_checked_batched_fp8(reduce):
    dev = GH.device()
    cfg = W.BATCHED_FP8.scaled(name="chk_batched", M=96, H=256, I=256, E=8, top_k=2)
    inp = W.make_inputs(cfg, 5160 + int(reduce))
    print(f"[case] checked batched fp8 reduce={reduce}", flush=True)
    (out_r, ws_r, info_r), (out_c, ws_c, info_c) = _both(
        lambda: GH.run_batched(inp, dev, reduce=reduce, out_dtype=torch.float32, packed=True))
    assert B.device_status(ws_c, info_c) == 0
    if reduce:
        assert torch.equal(out_r, out_c)
    else:                               # rows past the counts are never written
        rows = torch.as_tensor(GH.batched_rows(inp)[0], device=dev)
        assert torch.equal(out_r.reshape(-1, cfg.H)[rows], out_c.reshape(-1, cfg.H)[rows])
