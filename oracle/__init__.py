"""CPU oracle for the bit-nested W4/W8 quantized linear (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``bitnest_oracle.c`` (plain C, fp64 / int64, compiled
with gcc ``-O2 -ffp-contract=off``, no fast-math); this module only builds it
and marshals numpy arrays. What each function computes, and the passage of the
BitNest-Llama-3-8B model card it follows, is written in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnest_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt copy of this same source (for instance one compiled with
# sanitizers) may be named here; it is then loaded as it is, never rebuilt.
_LIB_OVERRIDE = os.environ.get("BITNEST_ORACLE_LIB")
GROUP = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU involved). Returns the library path."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-D_GNU_SOURCE", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_unpack_plane.argtypes = [P, I, I, P]
        lib.oracle_quant_act.argtypes = [P, I, I, I, P, P]
        lib.oracle_partials.argtypes = [P, P, P, I, I, I, P, P, P, I]
        lib.oracle_dequant.argtypes = [I, P, P, P, I, I, P]
        lib.oracle_linear.argtypes = [I, P, P, I, P, P, P, I, I, I, P, I]
        lib.oracle_hadamard_rotate.argtypes = [P, I, I, I, P]
        lib.oracle_pack_nested.argtypes = [P, I, I, P, P, P]
        lib.oracle_greedy_accept.argtypes = [P, I, I, P, P, P, P]
        lib.oracle_kv_attention.argtypes = [P, I, I, I, I, P, P, P, P, P, P, P, I]
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_max_threads.argtypes = []
        for f in ("oracle_unpack_plane", "oracle_quant_act", "oracle_partials",
                  "oracle_dequant", "oracle_linear", "oracle_hadamard_rotate", "oracle_pack_nested",
                  "oracle_greedy_accept", "oracle_kv_attention", "oracle_max_threads"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _check(rc, what):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (what, rc))


def max_threads() -> int:
    return _load().oracle_max_threads()


def half_to_double(bits: int) -> float:
    """IEEE binary16 bit pattern -> float, decoded from the format's definition."""
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def unpack_plane(plane: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N, K/2] plane -> unsigned nibbles uint8 [N, K] (column 2j = low nibble)."""
    plane = _c(plane, np.uint8)
    N = plane.shape[0]
    if plane.shape != (N, K // 2):
        raise ValueError("plane shape %s does not match K=%d" % (plane.shape, K))
    u = np.empty((N, K), np.uint8)
    _check(_load().oracle_unpack_plane(_ptr(plane), N, K, _ptr(u)), "unpack_plane")
    return u


def quant_act(x: np.ndarray, act_group: int = 0):
    """fp32 [M, K] -> (int8 codes [M, K], fp32 scales [M] or [M, K/128])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    S = 1 if act_group == 0 else K // GROUP
    s = np.empty((M, S), np.float32)
    _check(_load().oracle_quant_act(_ptr(x), M, K, act_group, _ptr(q), _ptr(s)), "quant_act")
    return q, (s[:, 0].copy() if act_group == 0 else s)


def partials(q: np.ndarray, hi: np.ndarray, lo: np.ndarray | None = None, threads: int = 0):
    """Exact per-group integer partials int32 [M, N, K/128].

    Returns P_hi for the draft, or (P_hi, P_lo, P8) when ``lo`` is given.
    """
    q = _c(q, np.int8)
    hi = _c(hi, np.uint8)
    M, K = q.shape
    N = hi.shape[0]
    if hi.shape != (N, K // 2):
        raise ValueError("hi shape mismatch")
    G = K // GROUP
    p_hi = np.empty((M, N, G), np.int32)
    p_lo = p8 = None
    if lo is not None:
        lo = _c(lo, np.uint8)
        if lo.shape != hi.shape:
            raise ValueError("lo shape mismatch")
        p_lo = np.empty_like(p_hi)
        p8 = np.empty_like(p_hi)
    _check(_load().oracle_partials(_ptr(q), _ptr(hi), _ptr(lo), M, N, K, _ptr(p_hi),
                                   _ptr(p_lo), _ptr(p8), threads or max_threads()), "partials")
    return p_hi if lo is None else (p_hi, p_lo, p8)


def dequant(hi: np.ndarray, scale: np.ndarray, lo: np.ndarray | None = None) -> np.ndarray:
    """Dense dequantised weight fp64 [N, K]: draft if ``lo`` is None, else target."""
    hi = _c(hi, np.uint8)
    scale = _c(scale, np.uint16)
    N, half = hi.shape
    K = 2 * half
    if scale.shape != (N, K // GROUP):
        raise ValueError("scale shape mismatch")
    if lo is not None:
        lo = _c(lo, np.uint8)
    W = np.empty((N, K), np.float64)
    _check(_load().oracle_dequant(0 if lo is None else 1, _ptr(hi), _ptr(lo), _ptr(scale),
                                  N, K, _ptr(W)), "dequant")
    return W


def linear(q: np.ndarray, xs: np.ndarray, hi: np.ndarray, scale: np.ndarray,
           lo: np.ndarray | None = None, act_group: int = 0, threads: int = 0) -> np.ndarray:
    """y64 fp64 [M, N] = (q * s_a) @ W^T, dequantise-then-multiply; target if ``lo`` given."""
    q = _c(q, np.int8)
    xs = _c(xs, np.float32)
    hi = _c(hi, np.uint8)
    scale = _c(scale, np.uint16)
    M, K = q.shape
    N = hi.shape[0]
    if hi.shape != (N, K // 2) or scale.shape != (N, K // GROUP):
        raise ValueError("plane/scale shape mismatch")
    exp_xs = (M,) if act_group == 0 else (M, K // GROUP)
    if xs.shape != exp_xs:
        raise ValueError("xs shape %s, expected %s" % (xs.shape, exp_xs))
    if lo is not None:
        lo = _c(lo, np.uint8)
        if lo.shape != hi.shape:
            raise ValueError("lo shape mismatch")
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_linear(0 if lo is None else 1, _ptr(q), _ptr(xs), act_group, _ptr(hi),
                                 _ptr(lo), _ptr(scale), M, N, K, _ptr(y), threads or max_threads()),
           "linear")
    return y


def hadamard_rotate(x: np.ndarray, block: int) -> np.ndarray:
    """fp32 [M, K] -> fp32 [M, K]: each token's blocks of ``block`` columns
    times the normalised Sylvester-Hadamard matrix (the R4 reading in the C
    file's header: fp32 fast transform, stages 1, 2, ..., block/2, then one
    multiply by the fp32 value nearest 1/sqrt(block))."""
    x = _c(x, np.float32)
    M, K = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_hadamard_rotate(_ptr(x), M, K, int(block), _ptr(y)), "hadamard_rotate")
    return y


def hadamard_quant_act(x: np.ndarray, block: int):
    """The down_proj input path: R4 rotation, then per-token int8
    quantisation. Returns (codes int8 [M, K], scales fp32 [M], rotated fp32 [M, K])."""
    r = hadamard_rotate(x, block)
    q, s = quant_act(r, 0)
    return q, s, r


def float_to_half_bits(f: float) -> int:
    """fp32 value -> IEEE binary16 bit pattern, round to nearest even."""
    return int(_load().oracle_float_to_half(float(np.float32(f))))


def pack_nested(W: np.ndarray):
    """fp32 weights [N, K] -> (hi uint8 [N, K/2], lo uint8 [N, K/2], scale fp16 bits uint16
    [N, K/128]): the nested packing reading in the C file's header (symmetric 15-step RTN
    high nibble with fp16 scale amax/7.5, closed-form residual low nibble)."""
    W = _c(W, np.float32)
    N, K = W.shape
    hi = np.empty((N, K // 2), np.uint8)
    lo = np.empty((N, K // 2), np.uint8)
    sc = np.empty((N, K // GROUP), np.uint16)
    _check(_load().oracle_pack_nested(_ptr(W), N, K, _ptr(hi), _ptr(lo), _ptr(sc)), "pack_nested")
    return hi, lo, sc


def greedy_accept(logits: np.ndarray, draft: np.ndarray):
    """Greedy verification: logits fp32 [gamma + 1, V], draft int32 [gamma] ->
    (target argmax per row int32 [gamma + 1], accepted count, next token)."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    draft = _c(np.asarray(draft, np.int32).reshape(-1), np.int32)
    if draft.shape != (R - 1,):
        raise ValueError("draft must hold gamma = R - 1 tokens")
    targ = np.empty(R, np.int32)
    n = np.zeros(1, np.int32)
    nxt = np.zeros(1, np.int32)
    _check(_load().oracle_greedy_accept(_ptr(logits), R, V, _ptr(draft) if R > 1 else None, _ptr(targ), _ptr(n),
                                        _ptr(nxt)), "greedy_accept")
    return targ, int(n[0]), int(nxt[0])


HEAD_DIM = 128


def kv_attention(q: np.ndarray, k_hi: np.ndarray, k_scale: np.ndarray, v_hi: np.ndarray, v_scale: np.ndarray,
                 k_lo: np.ndarray | None = None, v_lo: np.ndarray | None = None, threads: int = 0) -> np.ndarray:
    """Decode attention over a nested KV cache (the reading in the C file's
    header): q fp32 [M, Hq, 128]; planes uint8 [T, Hkv, 64]; scales fp16 bits
    uint16 [T, Hkv]; KV4 without the lo planes, KV8 with them. -> fp64 [M, Hq, 128]."""
    q = _c(q, np.float32)
    M, Hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dimension must be 128")
    k_hi, v_hi = _c(k_hi, np.uint8), _c(v_hi, np.uint8)
    k_scale, v_scale = _c(k_scale, np.uint16), _c(v_scale, np.uint16)
    T, Hkv, half = k_hi.shape
    if half != HEAD_DIM // 2 or v_hi.shape != k_hi.shape or k_scale.shape != (T, Hkv) or v_scale.shape != (T, Hkv):
        raise ValueError("KV plane / scale shape mismatch")
    if (k_lo is None) != (v_lo is None):
        raise ValueError("give both lo planes or neither")
    if k_lo is not None:
        k_lo, v_lo = _c(k_lo, np.uint8), _c(v_lo, np.uint8)
        if k_lo.shape != k_hi.shape or v_lo.shape != k_hi.shape:
            raise ValueError("lo plane shape mismatch")
    out = np.empty((M, Hq, HEAD_DIM), np.float64)
    _check(_load().oracle_kv_attention(_ptr(q), M, Hq, Hkv, T, _ptr(k_hi), _ptr(k_lo), _ptr(k_scale), _ptr(v_hi),
                                       _ptr(v_lo), _ptr(v_scale), _ptr(out), threads or max_threads()),
           "kv_attention")
    return out
