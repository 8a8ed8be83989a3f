"""CPU oracle for the fused MoE forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and shares no
code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision);
this module only builds it with gcc and marshals numpy / torch CPU arrays.
Each C function's header comment cites the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, FP8 = 0, 1, 2
U8, U4 = 3, 4                    # WNA16 weight codes (8 or 4 bits)
SOFTMAX, SIGMOID = 0, 1
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8}


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Routing(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("scoring", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("group_count", ctypes.c_int32), ("k_group", ctypes.c_int32),
                ("group_select_mode", ctypes.c_int32), ("logits_dtype", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_double)]


class _Experts(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("bias_dtype", ctypes.c_int32), ("w13_bias", ctypes.c_void_p),
                ("w2_bias", ctypes.c_void_p), ("requant_z", ctypes.c_int32),
                ("block", ctypes.c_int32), ("group", ctypes.c_int32),
                ("w13_zero", ctypes.c_void_p), ("w2_zero", ctypes.c_void_p),
                ("wq_bf16", ctypes.c_int32), ("z_bf16", ctypes.c_int32)]


class _Acts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("quantize", ctypes.c_int32),
                ("block", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_decode.restype = ctypes.c_double
    lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
    lib.oracle_fp8_encode.restype = ctypes.c_uint8
    lib.oracle_quant_row_fp8.argtypes = [P, i64, P, P]
    lib.oracle_quant_row_fp8.restype = None
    lib.oracle_quant_row_fp8_groups.argtypes = [P, i64, i64, P, P]
    lib.oracle_quant_row_fp8_groups.restype = None
    lib.oracle_route.argtypes = [ctypes.POINTER(_Routing), P, i64, P, P]
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_group_keys.argtypes = [ctypes.POINTER(_Routing), P, i64, P]
    lib.oracle_group_keys.restype = ctypes.c_int
    lib.oracle_align.argtypes = [P, i64, i32, i32, P, P, i64, P, i64, P]
    lib.oracle_align.restype = ctypes.c_int
    lib.oracle_forward_tokens.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts), i32,
                                          P, P, P, i64, P, i32, P, i32]
    lib.oracle_forward_tokens.restype = ctypes.c_int
    lib.oracle_expert_rows.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts), P, P,
                                       i64, P, i32]
    lib.oracle_expert_rows.restype = ctypes.c_int
    lib.oracle_unpack_wq.argtypes = [i32, i32, i64, i64, i64, i64, P, P, i32, P, P]
    lib.oracle_unpack_wq.restype = ctypes.c_int
    lib.oracle_fp8_tie_alt.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.oracle_fp8_tie_alt.restype = ctypes.c_int
    lib.oracle_max_ties.argtypes = []
    lib.oracle_max_ties.restype = ctypes.c_int
    lib.oracle_forward_tokens_ties.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts),
                                               i32, P, P, P, i64, P, i32, P, i32,
                                               ctypes.c_float, P, P]
    lib.oracle_forward_tokens_ties.restype = ctypes.c_int
    lib.oracle_expert_rows_ties.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts), P,
                                            P, i64, P, i32, ctypes.c_float, P, P]
    lib.oracle_expert_rows_ties.restype = ctypes.c_int
    lib.oracle_expert_z_codes.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts), P, P,
                                          i64, ctypes.c_float, P, P, P, i32]
    lib.oracle_expert_z_codes.restype = ctypes.c_int
    lib.oracle_expert_z.argtypes = [ctypes.POINTER(_Experts), ctypes.POINTER(_Acts), P, P, i64,
                                    P, i32]
    lib.oracle_expert_z.restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling

def _np(x, want=None):
    """torch (CPU) or numpy -> contiguous numpy, bf16 as uint16 bits, fp8 as uint8 codes."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            elif x.dtype == torch.float8_e4m3fn:
                x = x.view(torch.uint8).numpy()
            else:
                x = x.numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if want is not None:
        x = np.ascontiguousarray(x, dtype=want)
    return x


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


# ---------------------------------------------------------------- scalar formats

def fp8_decode(codes) -> np.ndarray:
    lib = load()
    c = _np(codes, np.uint8)
    return np.array([lib.oracle_fp8_decode(int(v)) for v in c.ravel()]).reshape(c.shape)


def fp8_encode(x) -> np.ndarray:
    lib = load()
    a = _np(x, np.float32)
    return np.array([lib.oracle_fp8_encode(float(v)) for v in a.ravel()],
                    dtype=np.uint8).reshape(a.shape)


def quant_rows_fp8(x, block=0):
    """Dynamic fp8 of each row: returns (codes uint8 [R, H], scales float32).
    block 0: one scale per row, [R]; block B > 0: one per B columns,
    [R, ceil(H / B)] (the block-wise granularity of "FP8 W8A8")."""
    lib = load()
    a = _np(x, np.float32)
    R, H = a.shape
    q = np.empty((R, H), np.uint8)
    if block:
        s = np.empty((R, -(-H // block)), np.float32)
        for r in range(R):
            row = np.ascontiguousarray(a[r])
            lib.oracle_quant_row_fp8_groups(row.ctypes.data, H, block, q[r].ctypes.data,
                                            s[r].ctypes.data)
        return q, s
    s = np.empty(R, np.float32)
    for r in range(R):
        row = np.ascontiguousarray(a[r])
        lib.oracle_quant_row_fp8(row.ctypes.data, H, q[r].ctypes.data, s[r:].ctypes.data)
    return q, s


# ---------------------------------------------------------------- routing / align

def _routing(E, top_k, scoring, renormalize, group_count, k_group, group_select_mode, rsf,
             logits_dtype):
    return _Routing(E, top_k, SIGMOID if scoring == "sigmoid" else SOFTMAX, int(renormalize),
                    group_count, k_group, group_select_mode, logits_dtype, float(rsf))


def route(logits, top_k, scoring="softmax", renormalize=False, group_count=1, k_group=1,
          group_select_mode=0, routed_scaling_factor=1.0):
    """Returns (topk_ids int32 [M, k], topk_weights float64 [M, k])."""
    lib = load()
    lg = _np(logits)
    M, E = lg.shape
    R = _routing(E, top_k, scoring, renormalize, group_count, k_group, group_select_mode,
                 routed_scaling_factor, _dtype_code(lg))
    ids = np.empty((M, top_k), np.int32)
    w = np.empty((M, top_k), np.float64)
    rc = lib.oracle_route(ctypes.byref(R), lg.ctypes.data, M, ids.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_route rejected the routing parameters")
    return ids, w


def group_keys(logits, group_count, group_select_mode, scoring="softmax"):
    lib = load()
    lg = _np(logits)
    M, E = lg.shape
    R = _routing(E, 1, scoring, 0, group_count, 1, group_select_mode, 1.0, _dtype_code(lg))
    keys = np.empty((M, group_count), np.float32)
    lib.oracle_group_keys(ctypes.byref(R), lg.ctypes.data, M, keys.ctypes.data)
    return keys


def align(topk_ids, E, block_m, expert_map=None):
    """Returns (counts [E], sorted_ids [num_post_padded], expert_ids [npp/BM], npp).
    expert_map [global experts]: topk_ids are global ids, mapped to the E
    local experts; items of experts mapped to -1 get no row."""
    lib = load()
    ids = _np(topk_ids, np.int32).ravel()
    if expert_map is not None:
        ids = np.ascontiguousarray(_np(expert_map, np.int32)[ids], dtype=np.int32)
    Mk = ids.size
    cap = Mk + E * (block_m - 1)
    counts = np.empty(E, np.int32)
    sorted_ids = np.empty(max(cap, 1), np.int32)
    expert_ids = np.empty(max(cap // block_m + 1, 1), np.int32)
    npp = np.zeros(1, np.int32)
    rc = lib.oracle_align(ids.ctypes.data, Mk, E, block_m, counts.ctypes.data,
                          sorted_ids.ctypes.data, cap, expert_ids.ctypes.data,
                          expert_ids.size, npp.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_align: id out of range")
    n = int(npp[0])
    return counts, sorted_ids[:n].copy(), expert_ids[: n // block_m].copy(), n


# ---------------------------------------------------------------- GPTQ / AWQ codes

GPTQ, AWQ = 1, 2


def unpack_wq(fmt: str, bits: int, qweight, qzeros=None, K=None, N=None, group=128,
              zero_adjust=0):
    """GPTQ- or AWQ-packed int32 codes of E experts -> the oracle's plain
    WNA16 codes ([E, K, N] bytes for 8 bits, [E, K, N/2] two a byte for 4)
    and zero points [E, ceil(K/group), N] (or None).  fmt: "gptq" | "awq"."""
    lib = load()
    qw = _np(qweight).astype(np.int32, copy=False)
    qw = np.ascontiguousarray(qw)
    E = qw.shape[0]
    per = 32 // bits
    code = {"gptq": GPTQ, "awq": AWQ}[fmt]
    if K is None:
        K = qw.shape[1] * per if code == GPTQ else qw.shape[1]
    if N is None:
        N = qw.shape[2] if code == GPTQ else qw.shape[2] * 8
    codes = np.zeros((E, K, N if bits == 8 else N // 2), np.uint8)
    ng = -(-K // group)
    qz = None if qzeros is None else np.ascontiguousarray(_np(qzeros).astype(np.int32, copy=False))
    zeros = None if qz is None else np.empty((E, ng, N), np.uint8)
    rc = lib.oracle_unpack_wq(code, bits, E, K, N, group, qw.ctypes.data, _ptr(qz),
                              int(zero_adjust), codes.ctypes.data, _ptr(zeros))
    if rc != 0:
        raise ValueError("oracle_unpack_wq: unsupported layout")
    return codes, zeros


# ---------------------------------------------------------------- expert FFN

class Experts:
    """Keeps the numpy views alive while the C side holds raw pointers.
    fp8 weights: block 0 takes per-output-channel scales w13_scale [E, 2I],
    w2_scale [E, H]; block B > 0 one scale per B x B block, w13_scale
    [E, ceil(2I/B), ceil(H/B)], w2_scale [E, ceil(H/B), ceil(I/B)].
    WNA16 (bits 8 or 4): unsigned codes, w13 [E, H, 2I] / w2 [E, I, H] bytes
    (bits 4: two per byte along the last dim, even column in the low nibble,
    so [E, H, I] / [E, I, H/2]); scales [E, ceil(K/group), N] float; zero
    points the same shape as uint8, or None for 2^(bits-1).  wq_bf16: the
    dequantised weights (q - z) s formed in float32 and rounded to bf16 (the
    reading in which the dequantised weight is the compute type), instead of
    exact.  z_bf16: z held in bf16 before the second GEMM (without
    requant_z)."""

    def __init__(self, w13, w2, w13_scale=None, w2_scale=None, w13_bias=None, w2_bias=None,
                 requant_z=False, block=0, bits=0, group=128, w13_zero=None, w2_zero=None,
                 wq_bf16=False, z_bf16=False):
        self.w13, self.w2 = _np(w13), _np(w2)
        E, H, N = self.w13.shape
        if bits == 4:
            N *= 2
        I = N // 2
        w2_shape = (E, I, H // 2) if bits == 4 else (E, I, H)
        assert self.w2.shape == w2_shape, (self.w2.shape, w2_shape)
        self.z13 = None if w13_zero is None else _np(w13_zero, np.uint8)
        self.z2 = None if w2_zero is None else _np(w2_zero, np.uint8)
        self.w13_scale = None if w13_scale is None else _np(w13_scale, np.float32)
        self.w2_scale = None if w2_scale is None else _np(w2_scale, np.float32)
        self.b13 = None if w13_bias is None else _np(w13_bias)
        self.b2 = None if w2_bias is None else _np(w2_bias)
        bias_dt = F32
        for b in (self.b13, self.b2):
            if b is not None:
                bias_dt = _dtype_code(b)
        wd = {8: U8, 4: U4}[bits] if bits else _dtype_code(self.w13)
        if bits:
            assert self.w13.dtype == np.uint8 and self.w2.dtype == np.uint8
            ng = lambda k: -(-k // group)
            assert self.w13_scale.shape == (E, ng(H), N), self.w13_scale.shape
            assert self.w2_scale.shape == (E, ng(I), H), self.w2_scale.shape
            for z, sc in ((self.z13, self.w13_scale), (self.z2, self.w2_scale)):
                assert z is None or z.shape == sc.shape
        elif wd == FP8:
            assert self.w13_scale is not None and self.w2_scale is not None
            if block:
                nb = lambda n: -(-n // block)
                assert self.w13_scale.shape == (E, nb(N), nb(H)), self.w13_scale.shape
                assert self.w2_scale.shape == (E, nb(H), nb(I)), self.w2_scale.shape
            else:
                assert self.w13_scale.size == E * N and self.w2_scale.size == E * H
        self.s = _Experts(H, I, E, wd, _ptr(self.w13), _ptr(self.w2), _ptr(self.w13_scale),
                          _ptr(self.w2_scale), bias_dt, _ptr(self.b13), _ptr(self.b2),
                          int(requant_z), int(block), int(group), _ptr(self.z13),
                          _ptr(self.z2), int(wq_bf16), int(z_bf16))
        self.H, self.I, self.E = H, I, E


class Acts:
    """Activation rows.  fp8 codes come with scales [rows] (block 0) or
    [rows, ceil(H/B)] (block B); quantize=True quantises float rows the same
    way first."""

    def __init__(self, data, scale=None, quantize=False, block=0):
        self.data = _np(data)
        self.H = self.data.shape[-1]
        self.data = self.data.reshape(-1, self.H)
        self.scale = None if scale is None else _np(scale, np.float32).ravel()
        dt = _dtype_code(self.data)
        if dt == FP8:
            assert self.scale is not None
            groups = -(-self.H // block) if block else 1
            assert self.scale.size == self.data.shape[0] * groups, self.scale.size
        self.s = _Acts(dt, _ptr(self.data), _ptr(self.scale), int(quantize), int(block))


class Ties:
    """fp8 z codes decided within a relative window of a rounding tie, per
    output row: count[n] such codes, and delta[n, i] (i < min(count[n],
    MAX_TIES)) the change of output row n if code i were rounded the other
    way.  Either rounding of such a code is a correct result; the output is
    linear in z, so any subset of the deltas may be added."""

    def __init__(self, count: np.ndarray, delta: np.ndarray):
        self.count, self.delta = count, delta


def fp8_tie_alt(t: float, window: float) -> int:
    """The fp8 code across the rounding midpoint within `window` (relative)
    of t, or -1."""
    return int(load().oracle_fp8_tie_alt(float(t), float(window)))


def max_ties() -> int:
    return int(load().oracle_max_ties())


def forward_tokens(experts: Experts, acts: Acts, topk_ids, topk_w, tokens=None, nthreads=0,
                   expert_map=None, weight_on_input=False, tie_window=0.0):
    """y[n] = sum_j w[t,j] f_{id[t,j]}(x_t) for t = tokens[n]; float64 [n, H].
    expert_map [global experts]: ids are global and map to experts' rows, -1
    for experts held elsewhere (left out).  weight_on_input: w scales z_r and
    the expert outputs are summed unweighted.  Returns (y, threads_used), or
    (y, threads_used, Ties) with tie_window > 0 (fp8 experts)."""
    lib = load()
    emap = None if expert_map is None else _np(expert_map, np.int32)
    ids = _np(topk_ids, np.int32)
    w = _np(topk_w, np.float64)
    M, K = ids.shape
    tok = np.arange(M, dtype=np.int64) if tokens is None else _np(tokens, np.int64).ravel()
    y = np.empty((tok.size, experts.H), np.float64)
    if tie_window > 0:
        cnt = np.zeros(tok.size, np.int32)
        dl = np.zeros((tok.size, max_ties(), experts.H), np.float64)
        used = lib.oracle_forward_tokens_ties(ctypes.byref(experts.s), ctypes.byref(acts.s), K,
                                              ids.ctypes.data, w.ctypes.data, tok.ctypes.data,
                                              tok.size, y.ctypes.data, int(nthreads), _ptr(emap),
                                              int(bool(weight_on_input)), float(tie_window),
                                              cnt.ctypes.data, dl.ctypes.data)
        return y, used, Ties(cnt, dl)
    used = lib.oracle_forward_tokens(ctypes.byref(experts.s), ctypes.byref(acts.s), K,
                                     ids.ctypes.data, w.ctypes.data, tok.ctypes.data, tok.size,
                                     y.ctypes.data, int(nthreads), _ptr(emap),
                                     int(bool(weight_on_input)))
    return y, used


def expert_rows(experts: Experts, acts: Acts, rows, expert_of_row, nthreads=0, tie_window=0.0):
    """out[n] = f_{expert_of_row[n]}(activation row rows[n]); float64 [n, H].
    Returns (out, threads_used), or (out, threads_used, Ties) with
    tie_window > 0 (fp8 experts)."""
    lib = load()
    r = _np(rows, np.int64).ravel()
    e = _np(expert_of_row, np.int32).ravel()
    assert r.size == e.size
    out = np.empty((r.size, experts.H), np.float64)
    if tie_window > 0:
        cnt = np.zeros(r.size, np.int32)
        dl = np.zeros((r.size, max_ties(), experts.H), np.float64)
        used = lib.oracle_expert_rows_ties(ctypes.byref(experts.s), ctypes.byref(acts.s),
                                           r.ctypes.data, e.ctypes.data, r.size, out.ctypes.data,
                                           int(nthreads), float(tie_window), cnt.ctypes.data,
                                           dl.ctypes.data)
        return out, used, Ties(cnt, dl)
    used = lib.oracle_expert_rows(ctypes.byref(experts.s), ctypes.byref(acts.s), r.ctypes.data,
                                  e.ctypes.data, r.size, out.ctypes.data, int(nthreads))
    return out, used


def expert_z(experts: Experts, acts: Acts, rows, expert_of_row, nthreads=0):
    """z = SiLU(gate) * up of each (activation row, expert) pair before any
    requantisation; float64 [n, I]."""
    lib = load()
    r = _np(rows, np.int64).ravel()
    e = _np(expert_of_row, np.int32).ravel()
    assert r.size == e.size
    z = np.empty((r.size, experts.I), np.float64)
    lib.oracle_expert_z(ctypes.byref(experts.s), ctypes.byref(acts.s), r.ctypes.data,
                        e.ctypes.data, r.size, z.ctypes.data, int(nthreads))
    return z


def expert_z_codes(experts: Experts, acts: Acts, rows, expert_of_row, tie_window=0.0,
                   nthreads=0):
    """The fp8 path's re-quantised z of each (activation row, expert) pair:
    (codes uint8 [n, I], scales float32 [n, ceil(I/128)], alt int16 [n, I]),
    alt the other code of a code within tie_window of a rounding tie, else -1."""
    lib = load()
    r = _np(rows, np.int64).ravel()
    e = _np(expert_of_row, np.int32).ravel()
    assert r.size == e.size
    I = experts.I
    G = (I + 127) // 128
    codes = np.empty((r.size, I), np.uint8)
    scales = np.empty((r.size, G), np.float32)
    alt = np.empty((r.size, I), np.int16)
    lib.oracle_expert_z_codes(ctypes.byref(experts.s), ctypes.byref(acts.s), r.ctypes.data,
                              e.ctypes.data, r.size, float(tie_window), codes.ctypes.data,
                              scales.ctypes.data, alt.ctypes.data, int(nthreads))
    return codes, scales, alt
