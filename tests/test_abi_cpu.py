"""C ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, the ctypes mirrors match the header's struct layout,
and host-side validation returns the documented status codes before any
device work (so fake device pointers are never touched)."""
import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_ffn_router_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def test_library_exports_every_declared_function():
    lib = B.load()
    decl = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", open(HEADER).read(), re.M)
    assert set(decl) == set(B.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    for name in decl:
        assert re.search(rf"\bT {name}$", nm, re.M), name
    assert B.moe_version().count(".") == 2


def test_checked_build_matches_release_abi():
    """libmoe_checked.so (the bounds-checked build) exports the same entry
    points, says so in its version, imports no getenv, and sizes workspaces
    exactly as libmoe.so does."""
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_CHECKED_PATH], capture_output=True,
                        text=True, check=True).stdout
    for name in B.EXPORTED:
        assert re.search(rf"\bT {name}$", nm, re.M), name
    und = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_CHECKED_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", und)
    assert not B.moe_version().endswith("checked")
    probs = [_prob(M=96, H=256, I=1040, E=4, top_k=2),
             _prob(M=64, H=512, I=256, E=8, top_k=2, w_layout=B.MOE_W_PACKED,
                   w_dtype=B.MOE_FP8_E4M3FN, fp8_block=128)]
    release = [B.moe_workspace_shapes(p.c()) for p in probs]
    with B.checked_library():
        assert B.moe_version().endswith("checked")
        checked = [B.moe_workspace_shapes(p.c()) for p in probs]
    assert not B.moe_version().endswith("checked")
    for r, c in zip(release, checked):
        assert bytes(r) == bytes(c)


def test_device_status_bits_match_header():
    body = re.search(r"typedef enum \{(.*?)\} moe_device_status;", open(HEADER).read(), re.S)
    vals = dict(re.findall(r"(MOE_DEV_\w+)\s*=\s*(\d+)", body.group(1)))
    assert {k: int(v) for k, v in vals.items()} == {
        "MOE_DEV_ID_RANGE": B.MOE_DEV_ID_RANGE, "MOE_DEV_COUNT_CLAMPED": B.MOE_DEV_COUNT_CLAMPED,
        "MOE_DEV_ROWS_OVERFLOW": B.MOE_DEV_ROWS_OVERFLOW, "MOE_DEV_TOKEN_MAP": B.MOE_DEV_TOKEN_MAP,
        "MOE_DEV_BOUNDS": B.MOE_DEV_BOUNDS}


def test_struct_layout_matches_header(tmp_path):
    fields = {"moe_problem": B.moe_problem, "moe_workspace_info": B.moe_workspace_info,
              "moe_args": B.moe_args}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void){"]
    for st, cls in fields.items():
        lines.append(f'printf("{st} size %zu\\n", sizeof({st}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = dict(l.rsplit(" ", 1) for l in out.strip().splitlines())
    for st, cls in fields.items():
        assert int(got[f"{st} size"]) == ctypes.sizeof(cls), st
        for f, _ in cls._fields_:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, (st, f)


def _prob(**kw):
    base = dict(M=16, H=64, I=128, E=8, top_k=2, act_dtype=B.MOE_BF16, w_dtype=B.MOE_BF16,
                out_dtype=B.MOE_BF16, logits_dtype=B.MOE_BF16, renormalize=True)
    base.update(kw)
    return B.Problem(**base)


def _status(prob):
    info = B.moe_workspace_info()
    return B.load().moe_workspace_shapes(ctypes.byref(prob.c()), ctypes.byref(info))


@pytest.mark.parametrize("kw,status", [
    (dict(), B.MOE_OK),
    (dict(top_k=9), B.MOE_ERR_INVALID_ARG),                 # top_k in [1, E]
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(E=0), B.MOE_ERR_INVALID_ARG),
    (dict(M=-1), B.MOE_ERR_INVALID_ARG),
    (dict(group_count=3), B.MOE_ERR_INVALID_ARG),           # E % group_count
    (dict(group_count=4, k_group=5), B.MOE_ERR_INVALID_ARG),  # k_group in [1, G]
    (dict(group_count=4, k_group=0), B.MOE_ERR_INVALID_ARG),
    (dict(group_count=1, k_group=2), B.MOE_ERR_INVALID_ARG),
    (dict(group_count=4, k_group=1, top_k=3), B.MOE_ERR_INVALID_ARG),  # top_k > k_group*E/G
    (dict(group_count=8, k_group=2, group_select_mode=1), B.MOE_ERR_INVALID_ARG),  # 1 expert/group
    (dict(group_count=4, k_group=2, group_select_mode=2), B.MOE_ERR_INVALID_ARG),
    (dict(routing=7), B.MOE_ERR_INVALID_ARG),
    (dict(routed_scaling_factor=float("nan")), B.MOE_ERR_INVALID_ARG),
    (dict(H=72), B.MOE_ERR_UNSUPPORTED),                     # H % 16
    (dict(I=40), B.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),      # f32 act needs f32 weights/out
    (dict(act_dtype=B.MOE_F32, w_dtype=B.MOE_F32, out_dtype=B.MOE_F32), B.MOE_OK),
    (dict(w_dtype=B.MOE_FP8_E4M3FN), B.MOE_OK),
    (dict(w_dtype=B.MOE_FP8_E4M3FN, I=144), B.MOE_ERR_UNSUPPORTED),   # fp8 groups of 128
    (dict(act_dtype=B.MOE_FP8_E4M3FN, w_dtype=B.MOE_FP8_E4M3FN), B.MOE_ERR_UNSUPPORTED),
    (dict(routing=B.MOE_ROUTE_PRECOMPUTED, group_count=3), B.MOE_OK),  # routing params unused
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=0), B.MOE_ERR_INVALID_ARG),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=32, act_dtype=B.MOE_FP8_E4M3FN,
          w_dtype=B.MOE_FP8_E4M3FN), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED), B.MOE_OK),
    (dict(w_layout=2), B.MOE_ERR_INVALID_ARG),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN, I=144), B.MOE_ERR_UNSUPPORTED),
    (dict(w_layout=B.MOE_W_PACKED, act_dtype=B.MOE_F32, w_dtype=B.MOE_F32, out_dtype=B.MOE_F32),
     B.MOE_ERR_UNSUPPORTED),
    # expert-parallel shard: routing over global_experts, E local experts
    (dict(global_experts=32), B.MOE_OK),
    (dict(global_experts=4), B.MOE_ERR_INVALID_ARG),              # fewer than E
    (dict(global_experts=2048), B.MOE_ERR_UNSUPPORTED),
    (dict(global_experts=-1), B.MOE_ERR_INVALID_ARG),
    (dict(global_experts=12, top_k=10), B.MOE_OK),                # top_k bound is global
    (dict(global_experts=12, group_count=3, k_group=2), B.MOE_OK),   # groups split the global set
    (dict(global_experts=12, group_count=8, k_group=2), B.MOE_ERR_INVALID_ARG),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=8, global_experts=16), B.MOE_ERR_UNSUPPORTED),
    (dict(apply_weight_on_input=1), B.MOE_OK),
    (dict(apply_weight_on_input=2), B.MOE_ERR_INVALID_ARG),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=8, apply_weight_on_input=1), B.MOE_ERR_UNSUPPORTED),
    (dict(chunk_tokens=4), B.MOE_OK),
    (dict(chunk_tokens=-1), B.MOE_ERR_INVALID_ARG),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=8, chunk_tokens=4), B.MOE_ERR_UNSUPPORTED),
    # block-wise fp8 scales: 128 x 128 blocks, packed fp8 weights only
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN, fp8_block=128), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN, fp8_block=128, H=80), B.MOE_OK),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=32, act_dtype=B.MOE_FP8_E4M3FN,
          w_dtype=B.MOE_FP8_E4M3FN, w_layout=B.MOE_W_PACKED, fp8_block=128), B.MOE_OK),
    (dict(w_dtype=B.MOE_FP8_E4M3FN, fp8_block=128), B.MOE_ERR_UNSUPPORTED),      # plain layout
    (dict(w_layout=B.MOE_W_PACKED, fp8_block=128), B.MOE_ERR_UNSUPPORTED),       # bf16 weights
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN, fp8_block=64),
     B.MOE_ERR_UNSUPPORTED),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_FP8_E4M3FN, fp8_block=-128),
     B.MOE_ERR_INVALID_ARG),
    # WNA16: 8- / 4-bit codes with bf16 activations, packed only
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, H=80, I=48), B.MOE_OK),
    (dict(fmt=B.MOE_FMT_BATCHED, max_tokens=8, w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4),
     B.MOE_OK),
    (dict(w_dtype=B.MOE_U4), B.MOE_ERR_UNSUPPORTED),                       # plain layout
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8, act_dtype=B.MOE_F32, out_dtype=B.MOE_F32),
     B.MOE_ERR_UNSUPPORTED),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8, fp8_block=128), B.MOE_ERR_UNSUPPORTED),
    # per-call tuning hints: tile family (bf16 any, WNA16 the DMA ones), GEMM1 width
    (dict(tile_hint=B.MOE_TILE_DMA_160), B.MOE_OK),
    (dict(tile_hint=B.MOE_TILE_REG_16), B.MOE_OK),
    (dict(tile_hint=B.MOE_TILE_DMA_32, gemm1_wave_cols=2), B.MOE_OK),
    (dict(tile_hint=4), B.MOE_ERR_INVALID_ARG),
    (dict(tile_hint=8), B.MOE_ERR_INVALID_ARG),
    (dict(tile_hint=-1), B.MOE_ERR_INVALID_ARG),
    (dict(gemm1_wave_cols=3), B.MOE_ERR_INVALID_ARG),
    (dict(gemm1_wave_cols=4), B.MOE_OK),
    (dict(w_dtype=B.MOE_FP8_E4M3FN, tile_hint=B.MOE_TILE_DMA_160), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_F32, w_dtype=B.MOE_F32, out_dtype=B.MOE_F32,
          tile_hint=B.MOE_TILE_REG_16), B.MOE_ERR_UNSUPPORTED),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, tile_hint=B.MOE_TILE_DMA_64), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, tile_hint=B.MOE_TILE_REG_64),
     B.MOE_ERR_UNSUPPORTED),
    (dict(tile_hint=B.MOE_TILE_DMA_256), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8, tile_hint=B.MOE_TILE_DMA_256),
     B.MOE_ERR_UNSUPPORTED),
    # WNA16 scale groups of 32 / 64 / 128 K rows
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, wq_group=32), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8, wq_group=64), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U8, wq_group=128), B.MOE_OK),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, wq_group=16), B.MOE_ERR_UNSUPPORTED),
    (dict(w_layout=B.MOE_W_PACKED, w_dtype=B.MOE_U4, wq_group=256), B.MOE_ERR_UNSUPPORTED),
    (dict(wq_group=64), B.MOE_ERR_INVALID_ARG),                            # bf16 weights
])
def test_problem_validation(kw, status):
    assert _status(_prob(**kw)) == status


def test_workspace_layout_is_aligned_and_sized():
    for kw in [dict(), dict(M=4096, H=7168, I=2048, E=256, top_k=8),
               dict(w_dtype=B.MOE_FP8_E4M3FN, I=256),
               dict(fmt=B.MOE_FMT_BATCHED, max_tokens=64, w_dtype=B.MOE_FP8_E4M3FN, I=256,
                    batched_reduce=True)]:
        p = _prob(**kw)
        info = B.moe_workspace_shapes(p.c())
        offs = [getattr(info, f) for f, _ in B.moe_workspace_info._fields_ if f.startswith("off_")]
        assert all(o % 256 == 0 for o in offs)
        assert info.bytes >= max(offs)
        assert info.max_sorted_len >= min(p.M * p.top_k, p.E * max(p.max_tokens, 1)) + \
            p.E * (info.block_m - 1) or p.fmt == B.MOE_FMT_BATCHED
        assert info.max_blocks == info.max_sorted_len // info.block_m
        assert info.block_m == 16


def test_expert_runs_are_padded_to_16_rows():
    for kw in [dict(M=32, H=2048, I=768, E=128, top_k=8), dict(M=512, H=4096, I=14336, E=8),
               dict(w_dtype=B.MOE_FP8_E4M3FN, I=256)]:
        info = B.moe_workspace_shapes(_prob(**kw).c())
        assert info.block_m == 16
        p = _prob(**kw)
        assert info.max_sorted_len == p.M * p.top_k + p.E * 15


def _args(**kw):
    fake = 4096   # never dereferenced: every case below fails validation on the host
    base = dict(hidden=fake, w13=fake, w2=fake, out=fake, router_logits=fake)
    base.update(kw)
    a = B.moe_args()
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,pkw,status", [
    (dict(router_logits=None), dict(), B.MOE_ERR_INVALID_ARG),
    (dict(hidden=None), dict(), B.MOE_ERR_INVALID_ARG),
    (dict(out=None), dict(), B.MOE_ERR_INVALID_ARG),
    (dict(), dict(has_w13_bias=True), B.MOE_ERR_INVALID_ARG),
    (dict(), dict(has_w2_bias=True), B.MOE_ERR_INVALID_ARG),
    (dict(), dict(routing=B.MOE_ROUTE_PRECOMPUTED), B.MOE_ERR_INVALID_ARG),
    (dict(), dict(w_dtype=B.MOE_FP8_E4M3FN), B.MOE_ERR_INVALID_ARG),      # scales missing
    (dict(), dict(fmt=B.MOE_FMT_BATCHED, max_tokens=8), B.MOE_ERR_INVALID_ARG),
    (dict(), dict(global_experts=32), B.MOE_ERR_INVALID_ARG),       # expert_map missing
    (dict(), dict(w_dtype=B.MOE_U4, w_layout=B.MOE_W_PACKED), B.MOE_ERR_INVALID_ARG),  # scales
    (dict(w13_scale=4096, w2_scale=4096, w13_zero=4096), dict(w_dtype=B.MOE_U8,
     w_layout=B.MOE_W_PACKED), B.MOE_ERR_INVALID_ARG),              # one zero-point grid only
])
def test_forward_rejects_missing_pointers(kw, pkw, status):
    p = _prob(**pkw).c()
    rc = B.moe_forward_status(p, _args(**kw), 1 << 20, 1 << 40, 0)
    assert rc == status


def test_forward_of_no_tokens_needs_no_token_arrays():
    """A contiguous forward with M = 0 reads and writes no token array: with
    hidden, out and the routing inputs null it returns MOE_OK before any
    device work (the same pointers are required as soon as M > 0)."""
    none = dict(hidden=None, out=None, router_logits=None)
    assert B.moe_forward_status(_prob(M=0).c(), _args(**none), 1 << 20, 1 << 40, 0) == B.MOE_OK
    assert B.moe_forward_status(_prob(M=1).c(), _args(**none), 1 << 20, 1 << 40, 0) == \
        B.MOE_ERR_INVALID_ARG


def test_forward_rejects_bad_workspace():
    p = _prob()
    info = B.moe_workspace_shapes(p.c())
    assert B.moe_forward_status(p.c(), _args(), 0, info.bytes, 0) == B.MOE_ERR_WORKSPACE
    assert B.moe_forward_status(p.c(), _args(), 256 * 1024 + 8, info.bytes, 0) == \
        B.MOE_ERR_WORKSPACE
    assert B.moe_forward_status(p.c(), _args(), 256 * 1024, info.bytes - 1, 0) == \
        B.MOE_ERR_WORKSPACE
    assert B.moe_status_string(B.MOE_ERR_WORKSPACE).startswith("workspace")


def test_packed_weight_sizes():
    """bf16: 16 KiB blocks of 64 rows x 128 columns: w13 ceil(I/64) x ceil(H/64)
    per expert (64 gate + 64 up columns a block), w2 ceil(H/128) x ceil(I/64).
    fp8: 16 KiB blocks of 128 columns x 128 K: w13 I/64 x ceil(H/128), w2
    ceil(H/128) x I/128."""
    for E, H, I in [(8, 4096, 14336), (2, 208, 176), (256, 7168, 2048), (1, 16, 16)]:
        b13, b2 = B.moe_packed_weight_bytes(_prob(E=E, H=H, I=I, top_k=1).c())
        blk = 64 * 128 * 2
        assert b13 == E * -(-I // 64) * -(-H // 64) * blk
        assert b2 == E * -(-H // 128) * -(-I // 64) * blk
    for E, H, I in [(64, 2048, 1408), (2, 208, 384), (1, 16, 128)]:
        b13, b2 = B.moe_packed_weight_bytes(
            _prob(E=E, H=H, I=I, top_k=1, w_dtype=B.MOE_FP8_E4M3FN).c())
        blk = 128 * 128
        assert b13 == E * (I // 64) * -(-H // 128) * blk
        assert b2 == E * -(-H // 128) * (I // 128) * blk
    # WNA16: blocks of 128 columns x 64 K codes (8 or 4 KiB): w13 ceil(I/64) x
    # ceil(H/64), w2 ceil(H/128) x ceil(I/64); the plain problem sizes them too
    for E, H, I in [(128, 2048, 768), (2, 80, 48), (1, 16, 16)]:
        for dt, blk in [(B.MOE_U8, 8192), (B.MOE_U4, 4096)]:
            for layout in (B.MOE_W_PLAIN, B.MOE_W_PACKED):
                b13, b2 = B.moe_packed_weight_bytes(
                    _prob(E=E, H=H, I=I, top_k=1, w_dtype=dt, w_layout=layout).c())
                assert b13 == E * -(-I // 64) * -(-H // 64) * blk
                assert b2 == E * -(-H // 128) * -(-I // 64) * blk
    for kw, status in [(dict(w_dtype=B.MOE_FP8_E4M3FN, I=144), B.MOE_ERR_UNSUPPORTED),
                       (dict(act_dtype=B.MOE_F32, w_dtype=B.MOE_F32, out_dtype=B.MOE_F32),
                        B.MOE_ERR_UNSUPPORTED),
                       (dict(H=72), B.MOE_ERR_UNSUPPORTED)]:
        b13, b2 = ctypes.c_size_t(), ctypes.c_size_t()
        rc = B.load().moe_packed_weight_bytes(ctypes.byref(_prob(**kw).c()), ctypes.byref(b13),
                                              ctypes.byref(b2))
        assert rc == status


def test_pack_rejects_null_pointers():
    fake = 4096   # never dereferenced: the null check fails first
    p = _prob().c()
    lib = B.load()
    assert lib.moe_pack_weights(ctypes.byref(p), None, fake, fake, fake, None) == \
        B.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(ctypes.byref(p), fake, fake, fake, None, None) == \
        B.MOE_ERR_INVALID_ARG


def test_chunked_workspace_is_sized_for_one_chunk():
    full = B.moe_workspace_shapes(_prob(M=4096, H=256, I=512, top_k=2).c())
    chunk = B.moe_workspace_shapes(_prob(M=4096, H=256, I=512, top_k=2, chunk_tokens=512).c())
    one = B.moe_workspace_shapes(_prob(M=512, H=256, I=512, top_k=2).c())
    assert chunk.bytes == one.bytes < full.bytes
    assert chunk.max_sorted_len == 512 * 2 + 8 * 15
    # a chunk larger than M is the unchunked problem
    big = B.moe_workspace_shapes(_prob(M=100, chunk_tokens=4096).c())
    assert big.bytes == B.moe_workspace_shapes(_prob(M=100).c()).bytes


def test_block_fp8_activation_scales_are_sized_per_group():
    """Block-wise fp8: the in-path activation scales take one float per row
    and 128 columns (a short last group included) instead of one per row."""
    kw = dict(M=64, H=320, I=256, w_dtype=B.MOE_FP8_E4M3FN, w_layout=B.MOE_W_PACKED)
    per_row = B.moe_workspace_shapes(_prob(**kw).c())
    per_blk = B.moe_workspace_shapes(_prob(fp8_block=128, **kw).c())
    span = lambda w: w.off_z - w.off_aq_scale          # the scale region (aligned to 256 B)
    assert span(per_row) >= 64 * 4
    assert span(per_blk) >= 64 * 3 * 4 > span(per_row)
    assert per_blk.off_aq_scale == per_row.off_aq_scale


def test_library_reads_no_environment():
    """No environment variable can change the library's choices: libmoe.so
    imports neither getenv nor secure_getenv."""
    und = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", und), "libmoe.so imports getenv"


def test_tile_hint_changes_only_what_it_names():
    """A tile hint may change the workspace (the chosen family decides the
    second GEMM's K split) but never the align metadata regions."""
    kw = dict(M=96, H=256, I=1040, E=4, top_k=2)
    auto = B.moe_workspace_shapes(_prob(**kw).c())
    forced = B.moe_workspace_shapes(_prob(tile_hint=B.MOE_TILE_DMA_160, **kw).c())
    reg = B.moe_workspace_shapes(_prob(tile_hint=B.MOE_TILE_REG_64, **kw).c())
    for f in ("off_topk_ids", "off_expert_counts", "off_sorted_ids", "off_expert_ids",
              "off_num_post_padded", "off_status", "off_z", "off_o"):
        assert getattr(auto, f) == getattr(forced, f) == getattr(reg, f), f
    assert forced.off_o2 != 0            # the 160-row family splits this GEMM2 in K
    assert reg.off_o2 == 0 and reg.bytes < forced.bytes


def test_status_word_has_its_own_region():
    for kw in [dict(), dict(fmt=B.MOE_FMT_BATCHED, max_tokens=64, batched_reduce=True),
               dict(fmt=B.MOE_FMT_BATCHED, max_tokens=64)]:
        info = B.moe_workspace_shapes(_prob(**kw).c())
        regions = sorted(getattr(info, f) for f, _ in B.moe_workspace_info._fields_
                         if f.startswith("off_") and getattr(info, f) != 0)
        assert info.off_status in regions and info.off_status % 256 == 0
        # no other region starts at the status word's offset (its 4 bytes are its own)
        assert regions.count(info.off_status) == 1 or info.off_status == 0


def test_static_entry_refuses_problems_beyond_its_array():
    """moe_forward_static sizes the problem on the host and refuses one whose
    workspace exceeds MOE_STATIC_WORKSPACE_BYTES before any device work
    (fake pointers are never touched); chunk_tokens brings it back in."""
    big = _prob(M=20000, H=1024, I=1024, top_k=2, routing=B.MOE_ROUTE_PRECOMPUTED)
    assert B.moe_workspace_shapes(big.c()).bytes > B.MOE_STATIC_WORKSPACE_BYTES
    args = _args(topk_ids=4096, topk_weights=4096)
    lib = B.load()
    assert lib.moe_forward_static(ctypes.byref(big.c()), ctypes.byref(args), None) == \
        B.MOE_ERR_STATIC_LIMIT
    assert "static" in B.moe_status_string(B.MOE_ERR_STATIC_LIMIT)
    big.chunk_tokens = 4096
    assert B.moe_workspace_shapes(big.c()).bytes <= B.MOE_STATIC_WORKSPACE_BYTES
    # argument errors come first, as in moe_forward
    assert lib.moe_forward_static(ctypes.byref(_prob(top_k=0).c()), ctypes.byref(args), None) \
        == B.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_static(ctypes.byref(_prob().c()), ctypes.byref(_args(hidden=None)),
                                  None) == B.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((1, 4, 2, 64, 32, 128), B.MOE_OK),
    ((2, 4, 2, 64, 32, 64), B.MOE_OK),
    ((1, 8, 2, 64, 32, 32), B.MOE_OK),
    ((2, 8, 2, 64, 32, 128), B.MOE_ERR_UNSUPPORTED),         # AWQ is 4-bit
    ((1, 2, 2, 64, 32, 128), B.MOE_ERR_UNSUPPORTED),
    ((3, 4, 2, 64, 32, 128), B.MOE_ERR_UNSUPPORTED),
    ((1, 4, 2, 64, 32, 100), B.MOE_ERR_UNSUPPORTED),
    ((1, 4, 2, 60, 32, 128), B.MOE_ERR_INVALID_ARG),         # GPTQ: K % 8
    ((2, 4, 2, 64, 36, 128), B.MOE_ERR_INVALID_ARG),         # AWQ: N % 8
    ((1, 4, 0, 64, 32, 128), B.MOE_ERR_INVALID_ARG),
])
def test_repack_validation(args, status):
    """Argument checks of moe_repack_wna16 on the host (OK cases are checked
    with null buffers, which fail before any device work)."""
    lib = B.load()
    fmt, bits, E, K, N, G = args
    fake = 4096                               # never dereferenced
    if status == B.MOE_OK:
        assert lib.moe_repack_wna16(fmt, bits, E, K, N, G, None, None, 0, fake, None,
                                    None) == B.MOE_ERR_INVALID_ARG
        assert lib.moe_repack_wna16(fmt, bits, E, K, N, G, fake, fake, 0, fake, None,
                                    None) == B.MOE_ERR_INVALID_ARG
    else:
        assert lib.moe_repack_wna16(fmt, bits, E, K, N, G, fake, None, 0, fake, None,
                                    None) == status
