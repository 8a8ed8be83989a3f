"""Seeded synthetic workloads for the fused MoE forward.

This module only draws random inputs of the shapes and distributions the
workloads name; it holds none of the method's arithmetic.  The HIP path and
the CPU oracle both consume the tensors it returns, already rounded to
their storage types, so parity never depends on the random generator.

Distribution notation: N(mu, v) takes the second argument as the variance
(fan-in initialisation N(0, 1/H) means standard deviation 1/sqrt(H)).

Two inputs are upstream of the fused MoE rather than part of it and are
prepared here with library calls only:
  * fp8 weights: per-output-channel scale amax/448 (or one per 128 x 128
    block) and a cast through torch.float8_e4m3fn (weights are quantised
    once, at load time);
  * the batched format's token layout: the dispatcher that produced it ran
    a top-k of (logits + per-expert offset) (torch.topk) and packed each
    expert's tokens in ascending token order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    M: int
    H: int
    I: int
    E: int
    top_k: int
    fmt: str = "contiguous"          # "contiguous" (M,K) or "batched" (E,max_tokens,K)
    act: str = "bf16"                # activation storage: f32 | bf16
    weight: str = "bf16"             # f32 | bf16 | fp8 (per-output-channel scales) |
                                     # u8 | u4 (WNA16 codes, group scales per 128 K rows)
    fp8_block: int = 0               # fp8: 128 = block-wise scales (128 x 128 weight
                                     # blocks, activations per token and 128 columns)
    wq_zero: bool = False            # u8 / u4 (WNA16): per-group zero points (asymmetric);
                                     # False: symmetric codes around 2^(bits-1)
    wq_group: int = 128              # u8 / u4 (WNA16): K rows per scale group (32, 64, 128)
    scoring: str = "softmax"         # softmax | sigmoid
    renormalize: bool = True
    group_count: int = 1
    k_group: int = 1
    group_select_mode: int = 0
    routed_scaling_factor: float = 1.0
    bias: bool = False
    expert_bias_var: float = 0.0     # per-expert logit offset ~ N(0, var)
    zipf_s: float = 0.0              # per-expert logit offset -s*ln(rank+1)
    max_tokens: int = 0              # batched: rows per expert slab (0 = M)
    local_experts: int = 0           # > 0: an expert-parallel shard holding experts
                                     # [0, local_experts) of the E routed over

    @property
    def logits_dtype(self) -> str:
        return "f32" if self.act == "f32" else "bf16"

    @property
    def out_dtype(self) -> str:
        return "f32" if self.act == "f32" else "bf16"

    def routed_rows(self) -> int:
        return self.M * self.top_k

    def flops(self, valid_rows: Optional[int] = None) -> float:
        """Algorithmic FLOPs of the two expert contractions."""
        rows = self.routed_rows() if valid_rows is None else valid_rows
        return 2.0 * rows * 3.0 * self.H * self.I

    def scaled(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Shapes follow the pages' examples: Mixtral-like
# (MindIE-SD single-card example: H 4096, I 14336, E 8, top-2) and
# DeepSeek-V3-like (MoonEP notation table: H 7168, H' 2048, E 256, top-8).
TINY_F32 = MoeConfig("tiny_f32", M=16, H=64, I=128, E=8, top_k=2, act="f32", weight="f32")
MIXTRAL_PREFILL = MoeConfig("mixtral_prefill_bf16", M=512, H=4096, I=14336, E=8, top_k=2)
DECODE_SMALL_EXPERTS = MoeConfig("decode_e128_bf16", M=32, H=2048, I=768, E=128, top_k=8)
DEEPSEEK_GROUPED = MoeConfig("deepseek_grouped_sigmoid_bf16", M=4096, H=7168, I=2048, E=256,
                             top_k=8, scoring="sigmoid", renormalize=False, group_count=8,
                             k_group=4, group_select_mode=1, routed_scaling_factor=2.5,
                             bias=True, expert_bias_var=0.5)
BATCHED_FP8 = MoeConfig("batched_fp8_skewed", M=8192, H=2048, I=1408, E=64, top_k=6,
                        fmt="batched", weight="fp8", renormalize=False, zipf_s=1.1)

CONFIGS = [TINY_F32, MIXTRAL_PREFILL, DECODE_SMALL_EXPERTS, DEEPSEEK_GROUPED, BATCHED_FP8]

# One rank of the DeepSeek-like layer under 8-way expert parallelism: the
# tokens of all 8 ranks (8 x 4096) are routed over the 256 experts and this
# rank holds 32 of them, about 1024 rows each (the MFMA-bound share).
EP8_SHARD = DEEPSEEK_GROUPED.scaled(name="ep8_shard_deepseek_bf16", M=32768, local_experts=32)

# The DeepSeek-like layer with block-wise fp8 weights (one scale per 128 x 128
# block, activations quantised per token and 128 columns in the path): the
# form DeepSeek-V3-class checkpoints ship.
DEEPSEEK_BLOCKFP8 = DEEPSEEK_GROUPED.scaled(name="deepseek_blockfp8", weight="fp8", fp8_block=128)

# Decode with WNA16 weights (the decode-sized layer of C3): 4-bit codes with
# symmetric groups (GPTQ-style default zero point 8), and 8-bit codes with
# per-group zero points.
DECODE_W4A16 = DECODE_SMALL_EXPERTS.scaled(name="decode_e128_w4a16", weight="u4")
DECODE_W8A16 = DECODE_SMALL_EXPERTS.scaled(name="decode_e128_w8a16", weight="u8", wq_zero=True)

# The Mixtral-shaped layer at M = 4096 tokens (about 1024 rows per expert):
# the compute-bound bf16 prefill shape (the M = 512 shape streams weights).
MIXTRAL_M4096 = MIXTRAL_PREFILL.scaled(name="mixtral_prefill_m4096_bf16", M=4096)

EXTRA = [EP8_SHARD, DEEPSEEK_BLOCKFP8, DECODE_W4A16, DECODE_W8A16, MIXTRAL_M4096]
BY_NAME = {c.name: c for c in CONFIGS + EXTRA}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _randn(shape, gen, device, std=1.0, dtype=torch.float32):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def quantize_weight_fp8(w: torch.Tensor):
    """Per-output-channel (last dim) fp8 e4m3fn codes + float32 scales.
    w: [E, K, N] float32 -> (codes float8_e4m3fn [E, K, N], scale [E, N])."""
    amax = w.abs().amax(dim=1)                                   # [E, N]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (w / scale[:, None, :]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes, scale.to(torch.float32)


def quantize_weight_fp8_blocks(w: torch.Tensor, B: int = 128):
    """Block-wise fp8 e4m3fn codes + one float32 scale (amax / 448, 1 for an
    all-zero block) per B x B block.  w: [E, K, N] float32 -> (codes
    float8_e4m3fn [E, K, N], scale [E, ceil(N / B), ceil(K / B)]), the scale
    grid indexed (output-column block, K block).  One expert at a time."""
    E, K, N = w.shape
    nk, nn = -(-K // B), -(-N // B)
    codes = torch.empty(E, K, N, dtype=torch.float8_e4m3fn, device=w.device)
    scale = torch.empty(E, nn, nk, dtype=torch.float32, device=w.device)
    for e in range(E):
        wp = torch.nn.functional.pad(w[e], (0, nn * B - N, 0, nk * B - K))
        amax = wp.abs().view(nk, B, nn, B).amax(dim=(1, 3))            # [nk, nn]
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (wp.view(nk, B, nn, B) / sc[:, None, :, None]).clamp_(-448.0, 448.0)
        codes[e] = q.view(nk * B, nn * B)[:K, :N].to(torch.float8_e4m3fn)
        scale[e] = sc.t()
    return codes, scale


def quantize_weight_wna16(w: torch.Tensor, bits: int, zero: bool, G: int = 128):
    """WNA16 codes of w [E, K, N] float32, one scale (and zero point) per G
    K rows and column: symmetric s = amax / (2^(bits-1) - 1) around the
    default zero point 2^(bits-1), or asymmetric s = (max - min) / (2^bits - 1)
    with z = round(-min / s).  Returns (codes uint8 [E, K, N], or two per byte
    along N for 4 bits [E, K, N / 2]; scale float32 [E, ceil(K/G), N]; zero
    uint8 of the same shape, or None)."""
    E, K, N = w.shape
    ng = -(-K // G)
    qmax = 2 ** bits - 1
    wp = torch.nn.functional.pad(w, (0, 0, 0, ng * G - K)).view(E, ng, G, N)
    if zero:
        lo, hi = wp.amin(dim=2), wp.amax(dim=2)
        s = torch.where(hi > lo, (hi - lo) / qmax, torch.ones_like(hi))
        z = torch.round(-lo / s).clamp_(0, qmax)
    else:
        amax = wp.abs().amax(dim=2)
        s = torch.where(amax > 0, amax / (2 ** (bits - 1) - 1), torch.ones_like(amax))
        z = torch.full_like(s, 2 ** (bits - 1))
    q = torch.round(wp / s[:, :, None, :] + z[:, :, None, :]).clamp_(0, qmax)
    q = q.view(E, ng * G, N)[:, :K].to(torch.uint8)
    if bits == 4:
        q = q[..., 0::2] | (q[..., 1::2] << 4)
    return q.contiguous(), s.to(torch.float32), (z.to(torch.uint8) if zero else None)


def _draw_hidden_logits(cfg: MoeConfig, gen, device):
    """The first draws of every workload: hidden, then the router logits
    (+ per-expert offsets)."""
    M, H, E = cfg.M, cfg.H, cfg.E
    hidden = _randn((M, H), gen, device, dtype=_TORCH_DT[cfg.act])
    logits = _randn((M, E), gen, device)
    if cfg.expert_bias_var > 0:
        logits += _randn((E,), gen, device, std=math.sqrt(cfg.expert_bias_var))[None, :]
    if cfg.zipf_s > 0:
        perm = torch.randperm(E, generator=gen, device=device)
        offset = -cfg.zipf_s * torch.log(perm.to(torch.float32) + 1.0)
        logits += offset[None, :]
    return hidden, logits.to(_TORCH_DT[cfg.logits_dtype])


AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)      # AWQ word slot i holds column 8 c + AWQ_ORDER[i]


def pack_wq_checkpoint(codes: torch.Tensor, zeros, bits: int, fmt: str):
    """Packs one code per byte [E, K, N] (and zero points [E, ng, N], or
    None) into a checkpoint's int32 words, as the quantiser that wrote the
    checkpoint did: "gptq" packs 32 / bits rows of a column into a word
    ([E, K * bits / 32, N]) and zero points along N ([E, ng, N * bits / 32]);
    "awq" (4-bit) packs 8 columns of a row into a word in the order
    AWQ_ORDER ([E, K, N / 8]), zero points alike.  Slot i of a word is bits
    [bits * i, bits * (i + 1))."""
    per = 32 // bits
    c = codes.to(torch.int64)

    def along_last(t, order):
        t = t.reshape(*t.shape[:-1], t.shape[-1] // per, per)
        w = torch.zeros(t.shape[:-1], dtype=torch.int64)
        for i, col in enumerate(order):
            w |= t[..., col] << (bits * i)
        return w

    if fmt == "gptq":
        E, K, N = c.shape
        t = c.reshape(E, K // per, per, N)
        w = torch.zeros(E, K // per, N, dtype=torch.int64)
        for i in range(per):
            w |= t[:, :, i, :] << (bits * i)
        zw = None if zeros is None else along_last(zeros.to(torch.int64), range(per))
    elif fmt == "awq":
        assert bits == 4
        w = along_last(c, AWQ_ORDER)
        zw = None if zeros is None else along_last(zeros.to(torch.int64), AWQ_ORDER)
    else:
        raise ValueError(fmt)
    to32 = lambda t: None if t is None else ((t + 2 ** 31) % 2 ** 32 - 2 ** 31).to(torch.int32)
    return to32(w), to32(zw)


def make_logits(cfg: MoeConfig, seed: int, device="cpu") -> torch.Tensor:
    """The router logits make_inputs(cfg, seed, device) draws, without the
    weights (the same generator stream, so the same values on one device)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return _draw_hidden_logits(cfg, gen, device)[1]


def make_inputs(cfg: MoeConfig, seed: int, device="cpu") -> dict:
    """Draws every input of one forward.  Order of draws: hidden, logits
    (+ offsets), w13, w2, w13_bias, w2_bias."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    M, H, I, E = cfg.M, cfg.H, cfg.I, cfg.E
    act_dt = _TORCH_DT[cfg.act]
    out = {"cfg": cfg, "seed": seed}

    hidden, logits = _draw_hidden_logits(cfg, gen, device)

    w_dt = torch.float32 if cfg.weight in ("fp8", "u8", "u4") else _TORCH_DT[cfg.weight]
    if cfg.local_experts:                       # the shard's experts only
        E = cfg.local_experts
        emap = torch.full((cfg.E,), -1, dtype=torch.int32, device=device)
        emap[:E] = torch.arange(E, dtype=torch.int32, device=device)
        out["expert_map"] = emap
    w13 = _randn((E, H, 2 * I), gen, device, std=1.0 / math.sqrt(H), dtype=w_dt)
    w2 = _randn((E, I, H), gen, device, std=1.0 / math.sqrt(I), dtype=w_dt)
    if cfg.weight in ("u8", "u4"):
        bits = 8 if cfg.weight == "u8" else 4
        out["w13"], out["w13_scale"], out["w13_zero"] = quantize_weight_wna16(
            w13, bits, cfg.wq_zero, cfg.wq_group)
        del w13
        out["w2"], out["w2_scale"], out["w2_zero"] = quantize_weight_wna16(w2, bits, cfg.wq_zero,
                                                                           cfg.wq_group)
        del w2
    elif cfg.weight == "fp8":
        quant = quantize_weight_fp8_blocks if cfg.fp8_block else quantize_weight_fp8
        out["w13"], out["w13_scale"] = quant(w13)
        del w13
        out["w2"], out["w2_scale"] = quant(w2)
        del w2
    else:
        out["w13"], out["w2"] = w13, w2
    if cfg.bias:
        bdt = act_dt
        out["w13_bias"] = _randn((E, 2 * I), gen, device, std=0.1, dtype=bdt)
        out["w2_bias"] = _randn((E, H), gen, device, std=0.1, dtype=bdt)
    else:
        out["w13_bias"] = out["w2_bias"] = None

    if cfg.fmt == "batched":
        out.update(_batched_layout(cfg, hidden, logits))
    else:
        out["hidden"] = hidden
        out["logits"] = logits
    return out


def _batched_layout(cfg: MoeConfig, hidden: torch.Tensor, logits: torch.Tensor) -> dict:
    """Packs the tokens the way a dispatcher hands them to batched experts:
    slab e holds, in ascending token order, the tokens whose top-k (of the
    offset logits) contains e.  Rows past expert_num_tokens[e] are NaN."""
    E, M, K = cfg.E, cfg.M, cfg.top_k
    T = cfg.max_tokens or M
    lg = logits.float()
    ids = torch.topk(lg, K, dim=-1).indices.to(torch.int32)             # [M, K]
    probs = torch.softmax(lg, dim=-1)
    w = torch.gather(probs, 1, ids.long())
    if cfg.renormalize:
        w = w / w.sum(-1, keepdim=True)
    w = (w * cfg.routed_scaling_factor).to(torch.float32)
    flat = ids.reshape(-1).long()
    order = torch.sort(flat, stable=True).indices                       # routed items by expert
    counts = torch.bincount(flat, minlength=E)
    starts = torch.cumsum(counts, 0) - counts
    e_sorted = flat[order]
    slot = torch.arange(flat.numel(), device=flat.device) - starts[e_sorted]
    assert int(counts.max()) <= T, "max_tokens too small for this routing"
    xb = torch.full((E, T, cfg.H), float("nan"), dtype=hidden.dtype, device=hidden.device)
    xb[e_sorted, slot] = hidden[order // K]
    token_map = torch.empty(M * K, dtype=torch.int32, device=flat.device)
    token_map[order] = (e_sorted * T + slot).to(torch.int32)
    return {"hidden": xb, "expert_num_tokens": counts.to(torch.int32),
            "token_map": token_map.view(M, K), "token_map_w": w,
            "tokens": hidden, "topk_ids": ids, "max_tokens": T}
