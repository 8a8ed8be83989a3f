"""Thin ctypes binding of libmoe's C ABI (include/moe.h).

Argument marshalling only: every step of the forward runs in the HIP
kernels behind ``moe_forward``.  PyTorch supplies device memory and the
stream.  There is no fallback: if libmoe.so is missing or a call fails,
this module raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
LIB_CHECKED_PATH = os.path.join(_HERE, "libmoe_checked.so")

# enums of moe.h
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = 0, -1, -2, -3, -4
MOE_ERR_STATIC_LIMIT = -5
MOE_STATIC_WORKSPACE_BYTES = 128 << 20
MOE_F32, MOE_BF16, MOE_FP8_E4M3FN, MOE_U8, MOE_U4 = 0, 1, 2, 3, 4
MOE_ROUTE_SOFTMAX, MOE_ROUTE_SIGMOID, MOE_ROUTE_PRECOMPUTED = 0, 1, 2
MOE_FMT_CONTIGUOUS, MOE_FMT_BATCHED = 0, 1
MOE_W_PLAIN, MOE_W_PACKED = 0, 1
MOE_TILE_AUTO, MOE_TILE_DMA_160, MOE_TILE_REG_64, MOE_TILE_REG_16 = 0, 1, 2, 3
MOE_TILE_DMA_32, MOE_TILE_DMA_64, MOE_TILE_DMA_256 = 5, 6, 7
MOE_DEV_ID_RANGE, MOE_DEV_COUNT_CLAMPED, MOE_DEV_ROWS_OVERFLOW, MOE_DEV_TOKEN_MAP = 1, 2, 4, 8
MOE_DEV_BOUNDS = 16             # bounds-checked build only

EXPORTED = ("moe_workspace_shapes", "moe_forward", "moe_forward_timed", "moe_packed_weight_bytes",
            "moe_pack_weights", "moe_forward_static", "moe_repack_wna16", "moe_status_string",
            "moe_version")
MOE_WQ_GPTQ, MOE_WQ_AWQ = 1, 2
STAGES = ("router", "align", "quant", "gemm1", "gemm2", "reduce")


class moe_problem(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("M", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32), ("routing", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("group_count", ctypes.c_int32),
                ("k_group", ctypes.c_int32), ("group_select_mode", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("has_w13_bias", ctypes.c_int32),
                ("has_w2_bias", ctypes.c_int32), ("batched_reduce", ctypes.c_int32),
                ("w_layout", ctypes.c_int32), ("global_experts", ctypes.c_int32),
                ("apply_weight_on_input", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("fp8_block", ctypes.c_int32), ("tile_hint", ctypes.c_int32),
                ("gemm1_wave_cols", ctypes.c_int32), ("wq_group", ctypes.c_int32)]


class moe_workspace_info(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_size_t), ("block_m", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("max_sorted_len", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in (
            "off_topk_ids", "off_topk_weights", "off_expert_counts", "off_expert_offsets",
            "off_sorted_ids", "off_expert_ids", "off_num_post_padded", "off_aq", "off_aq_scale",
            "off_z", "off_z_scale", "off_o", "off_o2", "off_status")]


class moe_args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "hidden", "a_scale", "router_logits", "topk_ids", "topk_weights", "expert_num_tokens",
        "token_map", "token_map_w", "w13", "w2", "w13_bias", "w2_bias", "w13_scale", "w2_scale",
        "out", "expert_map", "w13_zero", "w2_zero")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None
_opened: dict = {}


def _open(path: str) -> ctypes.CDLL:
    """dlopens one build of the library and declares its entry points."""
    if path in _opened:
        return _opened[path]
    try:   # share torch's HIP runtime (same SONAME) when torch is present
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m mixture_experts_ffn_router_amd.build`")
    lib = ctypes.CDLL(path)
    lib.moe_workspace_shapes.argtypes = [ctypes.POINTER(moe_problem),
                                         ctypes.POINTER(moe_workspace_info)]
    lib.moe_workspace_shapes.restype = ctypes.c_int
    lib.moe_forward.argtypes = [ctypes.POINTER(moe_problem), ctypes.POINTER(moe_args),
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_timed.argtypes = [ctypes.POINTER(moe_problem), ctypes.POINTER(moe_args),
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_forward_timed.restype = ctypes.c_int
    lib.moe_packed_weight_bytes.argtypes = [ctypes.POINTER(moe_problem),
                                            ctypes.POINTER(ctypes.c_size_t),
                                            ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_packed_weight_bytes.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [ctypes.POINTER(moe_problem)] + [ctypes.c_void_p] * 5
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.moe_forward_static.argtypes = [ctypes.POINTER(moe_problem), ctypes.POINTER(moe_args),
                                       ctypes.c_void_p]
    lib.moe_forward_static.restype = ctypes.c_int
    lib.moe_repack_wna16.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 2 + [
        ctypes.c_int] + [ctypes.c_void_p] * 3
    lib.moe_repack_wna16.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    _opened[path] = lib
    return lib


def load() -> ctypes.CDLL:
    """Loads the in-tree libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def checked_library():
    """Runs the enclosed calls on the bounds-checked build, libmoe_checked.so
    (same ABI and results; indices taken from device data are checked against
    their buffers and a miss sets MOE_DEV_BOUNDS in the device status word)."""
    global _lib
    prev = load()
    _lib = _open(LIB_CHECKED_PATH)
    try:
        yield _lib
    finally:
        _lib = prev


def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_version() -> str:
    return load().moe_version().decode()


def moe_workspace_shapes(problem: moe_problem) -> moe_workspace_info:
    info = moe_workspace_info()
    rc = load().moe_workspace_shapes(ctypes.byref(problem), ctypes.byref(info))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_workspace_shapes")
    return info


def moe_forward(problem: moe_problem, args: moe_args, workspace: int, workspace_bytes: int,
                stream: int) -> None:
    rc = load().moe_forward(ctypes.byref(problem), ctypes.byref(args), ctypes.c_void_p(workspace),
                            workspace_bytes, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward")


def moe_forward_static(problem: moe_problem, args: moe_args, stream: int) -> None:
    """The allocation-free forward (workspace in the library's static array)."""
    rc = load().moe_forward_static(ctypes.byref(problem), ctypes.byref(args),
                                   ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward_static")


def moe_packed_weight_bytes(problem: moe_problem):
    b13, b2 = ctypes.c_size_t(), ctypes.c_size_t()
    rc = load().moe_packed_weight_bytes(ctypes.byref(problem), ctypes.byref(b13), ctypes.byref(b2))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_packed_weight_bytes")
    return int(b13.value), int(b2.value)


def moe_pack_weights(problem: moe_problem, w13: int, w2: int, w13_packed: int, w2_packed: int,
                     stream: int) -> None:
    rc = load().moe_pack_weights(ctypes.byref(problem), ctypes.c_void_p(w13), ctypes.c_void_p(w2),
                                 ctypes.c_void_p(w13_packed), ctypes.c_void_p(w2_packed),
                                 ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_pack_weights")


def moe_forward_timed(problem: moe_problem, args: moe_args, workspace: int,
                      workspace_bytes: int, stream: int, events) -> None:
    """events: sequence of 2 * len(STAGES) hipEvent_t handles (ints or None)."""
    arr = (ctypes.c_void_p * (2 * len(STAGES)))(*[e or None for e in events])
    rc = load().moe_forward_timed(ctypes.byref(problem), ctypes.byref(args),
                                  ctypes.c_void_p(workspace), workspace_bytes,
                                  ctypes.c_void_p(stream), arr)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward_timed")


def moe_forward_status(problem: moe_problem, args: moe_args, workspace: int,
                       workspace_bytes: int, stream: int) -> int:
    """moe_forward returning the raw status (for argument-validation tests)."""
    return load().moe_forward(ctypes.byref(problem), ctypes.byref(args),
                              ctypes.c_void_p(workspace), workspace_bytes,
                              ctypes.c_void_p(stream))


# ------------------------------------------------------------ torch marshalling

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return MOE_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


@dataclass
class Problem:
    """Python view of moe_problem."""
    M: int
    H: int
    I: int
    E: int
    top_k: int
    fmt: int = MOE_FMT_CONTIGUOUS
    max_tokens: int = 0
    act_dtype: int = MOE_BF16
    w_dtype: int = MOE_BF16
    out_dtype: int = MOE_BF16
    logits_dtype: int = MOE_BF16
    routing: int = MOE_ROUTE_SOFTMAX
    renormalize: bool = False
    group_count: int = 1
    k_group: int = 1
    group_select_mode: int = 0
    routed_scaling_factor: float = 1.0
    has_w13_bias: bool = False
    has_w2_bias: bool = False
    batched_reduce: bool = False
    w_layout: int = MOE_W_PLAIN
    global_experts: int = 0
    apply_weight_on_input: bool = False
    chunk_tokens: int = 0
    fp8_block: int = 0
    tile_hint: int = MOE_TILE_AUTO
    gemm1_wave_cols: int = 0
    wq_group: int = 0

    def c(self) -> moe_problem:
        return moe_problem(self.fmt, self.M, self.H, self.I, self.E, self.top_k, self.max_tokens,
                           self.act_dtype, self.w_dtype, self.out_dtype, self.logits_dtype,
                           self.routing, int(self.renormalize), self.group_count, self.k_group,
                           self.group_select_mode, float(self.routed_scaling_factor),
                           int(self.has_w13_bias), int(self.has_w2_bias),
                           int(self.batched_reduce), int(self.w_layout), int(self.global_experts),
                           int(self.apply_weight_on_input), int(self.chunk_tokens),
                           int(self.fp8_block), int(self.tile_hint), int(self.gemm1_wave_cols),
                           int(self.wq_group))


@dataclass
class PackedWeights:
    """bf16 or fp8 expert weights re-laid out once by moe_pack_weights (uint8
    device buffers) with the plain shapes and the dtype they came from."""
    w13: object
    w2: object
    E: int
    H: int
    I: int
    w_dtype: int = MOE_BF16


def pack_weights(w13, w2, wq_bits: int = 0) -> PackedWeights:
    """Packs plain bf16 or fp8 w13 [E, H, 2I] / w2 [E, I, H] on their device
    (one launch pair on the current stream).  wq_bits 8 / 4: WNA16 codes in
    uint8 tensors, 4-bit codes two per byte along the last dim ([E, H, I] /
    [E, I, H / 2])."""
    import torch
    E, H, N = w13.shape
    if wq_bits == 4:
        N *= 2
    I = N // 2
    w2_shape = (E, I, H // 2) if wq_bits == 4 else (E, I, H)
    if tuple(w2.shape) != w2_shape:
        raise ValueError(f"w2 shape {tuple(w2.shape)} does not match w13 {tuple(w13.shape)}")
    wdt = {8: MOE_U8, 4: MOE_U4}[wq_bits] if wq_bits else _dtype_code(w13)
    if wq_bits and (w13.dtype != torch.uint8 or w2.dtype != torch.uint8):
        raise TypeError("WNA16 codes are uint8 tensors")
    prob = Problem(M=0, H=H, I=I, E=E, top_k=1, act_dtype=MOE_BF16, w_dtype=wdt,
                   out_dtype=MOE_BF16).c()
    b13, b2 = moe_packed_weight_bytes(prob)
    p13 = torch.empty(b13, dtype=torch.uint8, device=w13.device)
    p2 = torch.empty(b2, dtype=torch.uint8, device=w13.device)
    moe_pack_weights(prob, _ptr(w13), _ptr(w2), p13.data_ptr(), p2.data_ptr(),
                     current_stream_handle(w13.device))
    return PackedWeights(p13, p2, E, H, I, wdt)


def repack_wna16(fmt: str, bits: int, qweight, qzeros=None, K=None, N=None, group=128,
                 zero_adjust=0):
    """GPTQ / AWQ checkpoint codes (int32 device tensors, [E, ...] as in
    moe.h) -> (plain WNA16 codes uint8, zero points uint8 [E, ceil(K/group), N]
    or None), ready for pack_weights(..., wq_bits=bits)."""
    import torch
    code = {"gptq": MOE_WQ_GPTQ, "awq": MOE_WQ_AWQ}[fmt]
    per = 32 // bits
    E = qweight.shape[0]
    if K is None:
        K = qweight.shape[1] * per if code == MOE_WQ_GPTQ else qweight.shape[1]
    if N is None:
        N = qweight.shape[2] if code == MOE_WQ_GPTQ else qweight.shape[2] * 8
    dev = qweight.device
    codes = torch.empty(E, K, N if bits == 8 else N // 2, dtype=torch.uint8, device=dev)
    zeros = None if qzeros is None else torch.empty(E, -(-K // group), N, dtype=torch.uint8,
                                                    device=dev)
    rc = load().moe_repack_wna16(code, bits, E, K, N, group, _ptr(qweight), _ptr(qzeros),
                                 int(zero_adjust), _ptr(codes), _ptr(zeros),
                                 ctypes.c_void_p(current_stream_handle(dev)))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_repack_wna16")
    return codes, zeros


def _weights(w13, w2):
    """(w13 tensor, w2 tensor, E, H, I, w_dtype code, layout) of plain or packed weights."""
    if isinstance(w13, PackedWeights):
        return w13.w13, w13.w2, w13.E, w13.H, w13.I, w13.w_dtype, MOE_W_PACKED
    E, H, N = w13.shape
    return w13, w2, E, H, N // 2, _dtype_code(w13), MOE_W_PLAIN


def make_args(hidden, w13, w2, out, router_logits=None, topk_ids=None, topk_weights=None,
              w13_bias=None, w2_bias=None, w13_scale=None, w2_scale=None, a_scale=None,
              expert_num_tokens=None, token_map=None, token_map_w=None,
              expert_map=None, w13_zero=None, w2_zero=None) -> moe_args:
    return moe_args(_ptr(hidden), _ptr(a_scale), _ptr(router_logits), _ptr(topk_ids),
                    _ptr(topk_weights), _ptr(expert_num_tokens), _ptr(token_map),
                    _ptr(token_map_w), _ptr(w13), _ptr(w2), _ptr(w13_bias), _ptr(w2_bias),
                    _ptr(w13_scale), _ptr(w2_scale), _ptr(out), _ptr(expert_map),
                    _ptr(w13_zero), _ptr(w2_zero))


def allocate_workspace(problem: Problem, device):
    """A device buffer of the size moe_workspace_shapes asks for (torch
    allocations are 256-byte aligned)."""
    import torch
    info = moe_workspace_shapes(problem.c())
    ws = torch.empty(max(int(info.bytes), 256), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws, info


def device_status(workspace, info: moe_workspace_info) -> int:
    """The device status word of the last forward on `workspace` (an OR of
    the MOE_DEV_* bits); synchronises through the device-to-host copy."""
    off = int(info.off_status)
    return int(workspace[off:off + 4].view(__import__("torch").int32).item())


def current_stream_handle(device=None) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fused_moe(hidden, w13, w2, router_logits=None, *, top_k: int, renormalize: bool = False,
              routing: str = "softmax", group_count: int = 1, k_group: int = 1,
              group_select_mode: int = 0, routed_scaling_factor: float = 1.0, w13_bias=None,
              w2_bias=None, topk_ids=None, topk_weights=None, w13_scale=None, w2_scale=None,
              out_dtype=None, out=None, workspace=None, expert_map=None,
              apply_weight_on_input=False, chunk_tokens=0, fp8_block=0, w13_zero=None,
              w2_zero=None, tile_hint=MOE_TILE_AUTO, gemm1_wave_cols=0, static=False,
              wq_group=0):
    """Contiguous-format forward on torch device tensors (the MindIE-SD
    page's fused_moe argument list, single device).  w13 may be a
    PackedWeights (then w2 is ignored).  expert_map [global experts] int32
    makes this device an expert-parallel shard holding the E experts of w13
    (routing over len(expert_map) experts).  fp8_block=128: block-wise fp8
    scales (w13_scale [E, 2I/128, ceil(H/128)], w2_scale [E, ceil(H/128),
    I/128]).  WNA16 weights come packed (pack_weights(..., wq_bits)) with
    group scales w13_scale [E, ceil(H/128), 2I] / w2_scale [E, ceil(I/128), H]
    and optional uint8 zero points of the same shapes.  tile_hint /
    gemm1_wave_cols force a GEMM tile family / GEMM1 width (moe_problem's
    tuning fields; 0 = the library's choice).  static=True runs the
    allocation-free entry point (moe_forward_static: the library's own
    device array as workspace; workspace and info are then None).  Returns
    (out, workspace tensor, workspace info)."""
    import torch
    M = hidden.shape[0]
    w13, w2, E, H, I, wdt, layout = _weights(w13, w2)
    if topk_ids is not None:
        route = MOE_ROUTE_PRECOMPUTED
        top_k = topk_ids.shape[1]
    else:
        route = {"softmax": MOE_ROUTE_SOFTMAX, "sigmoid": MOE_ROUTE_SIGMOID}[routing]
    act = _dtype_code(hidden)
    odt = out_dtype or (torch.float32 if act == MOE_F32 else torch.bfloat16)
    prob = Problem(M=M, H=H, I=I, E=E, top_k=top_k, act_dtype=act, w_dtype=wdt,
                   out_dtype=_dtype_code(torch.empty(0, dtype=odt)),
                   logits_dtype=_dtype_code(router_logits) if router_logits is not None else 0,
                   routing=route, renormalize=renormalize, group_count=group_count,
                   k_group=k_group, group_select_mode=group_select_mode,
                   routed_scaling_factor=routed_scaling_factor,
                   has_w13_bias=w13_bias is not None, has_w2_bias=w2_bias is not None,
                   w_layout=layout,
                   global_experts=0 if expert_map is None else int(expert_map.numel()),
                   apply_weight_on_input=apply_weight_on_input, chunk_tokens=chunk_tokens,
                   fp8_block=fp8_block, tile_hint=tile_hint, gemm1_wave_cols=gemm1_wave_cols,
                   wq_group=wq_group)
    if out is None:
        out = torch.empty(M, H, dtype=odt, device=hidden.device)
    args = make_args(hidden, w13, w2, out, router_logits=router_logits, topk_ids=topk_ids,
                     topk_weights=topk_weights, w13_bias=w13_bias, w2_bias=w2_bias,
                     w13_scale=w13_scale, w2_scale=w2_scale, expert_map=expert_map,
                     w13_zero=w13_zero, w2_zero=w2_zero)
    if static:
        moe_forward_static(prob.c(), args, current_stream_handle(hidden.device))
        return out, None, None
    if workspace is None:
        workspace, info = allocate_workspace(prob, hidden.device)
    else:
        info = moe_workspace_shapes(prob.c())
    moe_forward(prob.c(), args, workspace.data_ptr(), workspace.numel(),
                current_stream_handle(hidden.device))
    return out, workspace, info


def fused_moe_batched(hidden, expert_num_tokens, w13, w2, *, M: int = 0, top_k: int = 1,
                      a_scale=None, w13_scale=None, w2_scale=None, w13_bias=None, w2_bias=None,
                      token_map=None, token_map_w=None, out_dtype=None, out=None,
                      workspace=None, fp8_block=0, w13_zero=None, w2_zero=None,
                      tile_hint=MOE_TILE_AUTO, static=False, wq_group=0):
    """Batched-format forward: hidden [E, max_tokens, H] + expert_num_tokens [E].
    M, top_k (when M > 0) promise that the slabs hold at most M * top_k valid
    rows, which bounds the workspace (slabs that break the promise are not
    computed; the device status word reports it).  With token_map /
    token_map_w ([M, top_k]; -1 for a copy with no row here) the rows are
    also weighted and reduced into out [M, H]; otherwise out is
    [E, max_tokens, H]."""
    import torch
    E, T, H = hidden.shape
    w13, w2, _, _, I, wdt, layout = _weights(w13, w2)
    reduce = token_map is not None
    if reduce:
        M, top_k = token_map.shape
    odt = out_dtype or torch.bfloat16
    prob = Problem(M=M, H=H, I=I, E=E, top_k=top_k, fmt=MOE_FMT_BATCHED,
                   max_tokens=T, act_dtype=_dtype_code(hidden), w_dtype=wdt,
                   out_dtype=_dtype_code(torch.empty(0, dtype=odt)),
                   routing=MOE_ROUTE_PRECOMPUTED, has_w13_bias=w13_bias is not None,
                   has_w2_bias=w2_bias is not None, batched_reduce=reduce, w_layout=layout,
                   fp8_block=fp8_block, tile_hint=tile_hint, wq_group=wq_group)
    if out is None:
        shape = (M, H) if reduce else (E, T, H)
        out = torch.empty(shape, dtype=odt, device=hidden.device)
    args = make_args(hidden, w13, w2, out, a_scale=a_scale, expert_num_tokens=expert_num_tokens,
                     token_map=token_map, token_map_w=token_map_w, w13_bias=w13_bias,
                     w2_bias=w2_bias, w13_scale=w13_scale, w2_scale=w2_scale,
                     w13_zero=w13_zero, w2_zero=w2_zero)
    if static:
        moe_forward_static(prob.c(), args, current_stream_handle(hidden.device))
        return out, None, None
    if workspace is None:
        workspace, info = allocate_workspace(prob, hidden.device)
    else:
        info = moe_workspace_shapes(prob.c())
    moe_forward(prob.c(), args, workspace.data_ptr(), workspace.numel(),
                current_stream_handle(hidden.device))
    return out, workspace, info
