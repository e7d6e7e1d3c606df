"""Bit-nested W4/W8 quantized linear on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/bitnest.h`` (library
``libbitnest.so`` in this directory, built by ``build.py``). The functions
keep the C names and only marshal arguments: they check dtypes, shapes and
devices of torch tensors, pass their device pointers and torch's current
stream, and raise ``BitnestError`` on a non-zero status. Every step of the
computation runs in the HIP kernels; there is no CPU or PyTorch fallback, and
calling any of them without the built library raises at once.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BitnestError", "GROUP", "MAX_M", "MAX_K", "library_path", "lib",
    "bitnest_abi_version", "bitnest_status_string", "bitnest_quant_act",
    "bitnest_linear_draft", "bitnest_linear_target", "bitnest_linear_partials",
    "bitnest_quant_linear_draft", "bitnest_quant_linear_target",
    "bitnest_hadamard_quant_act", "bitnest_hadamard_quant_linear_draft", "bitnest_hadamard_quant_linear_target",
    "bitnest_pack_nested", "bitnest_greedy_accept", "bitnest_greedy_accept_workspace_bytes",
    "bitnest_greedy_accept_noalloc", "bitnest_kv_attention",
    "bitnest_kv_attention_workspace_bytes", "kv_pack", "bitnest_linear_chain", "LinearChain", "ChainLink",
    "bitnest_stream_read",
]

GROUP = 128
MAX_M = 32
MAX_K = 16384
MAX_ROT_BLOCK = 512

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libbitnest.so")

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, 1, 2, 3, 4

_lib = None


class BitnestError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: status %d (%s)" % (what, status, bitnest_status_string(status)))


def lib() -> ctypes.CDLL:
    """The loaded C library, with argument types declared. Raises if not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                "libbitnest.so is not built (%s); run `python -m w8_quantized_linear_amd.build` "
                "or __graft_entry__.build() first" % library_path)
        L = ctypes.CDLL(library_path)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.bitnest_abi_version.argtypes = []
        L.bitnest_abi_version.restype = I
        L.bitnest_status_string.argtypes = [I]
        L.bitnest_status_string.restype = ctypes.c_char_p
        L.bitnest_quant_act.argtypes = [P, I, I, I, P, P, P]
        L.bitnest_linear_draft.argtypes = [P, P, I, P, P, P, I, I, I, P]
        L.bitnest_linear_target.argtypes = [P, P, I, P, P, P, P, I, I, I, P]
        L.bitnest_linear_partials.argtypes = [P, P, P, P, P, P, I, I, I, P]
        L.bitnest_quant_linear_draft.argtypes = [P, I, P, P, P, P, P, I, I, I, P]
        L.bitnest_quant_linear_target.argtypes = [P, I, P, P, P, P, P, P, I, I, I, P]
        L.bitnest_hadamard_quant_act.argtypes = [P, I, I, I, P, P, P, P]
        L.bitnest_hadamard_quant_linear_draft.argtypes = [P, I, P, P, P, P, P, I, I, I, P]
        L.bitnest_hadamard_quant_linear_target.argtypes = [P, I, P, P, P, P, P, P, I, I, I, P]
        L.bitnest_pack_nested.argtypes = [P, I, I, P, P, P, P]
        L.bitnest_greedy_accept.argtypes = [P, I, I, P, P, P, P, ctypes.c_size_t, P]
        L.bitnest_greedy_accept_noalloc.argtypes = [P, I, I, P, P, P, P]
        L.bitnest_greedy_accept_workspace_bytes.argtypes = [I, I]
        L.bitnest_greedy_accept_workspace_bytes.restype = ctypes.c_size_t
        L.bitnest_kv_attention_workspace_bytes.argtypes = [I, I, I]
        L.bitnest_kv_attention_workspace_bytes.restype = ctypes.c_size_t
        L.bitnest_kv_attention.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.bitnest_linear_chain.argtypes = [P, P, I, I, ctypes.c_uint32, P, ctypes.c_size_t, P]
        L.bitnest_chain_workspace_bytes.argtypes = []
        L.bitnest_stream_read.argtypes = [P, ctypes.c_size_t, I, I, ctypes.c_uint32, P, P]
        L.bitnest_chain_workspace_bytes.restype = ctypes.c_size_t
        for f in ("bitnest_quant_act", "bitnest_linear_draft", "bitnest_linear_target",
                  "bitnest_linear_partials", "bitnest_quant_linear_draft", "bitnest_quant_linear_target",
                  "bitnest_hadamard_quant_act", "bitnest_hadamard_quant_linear_draft",
                  "bitnest_hadamard_quant_linear_target", "bitnest_pack_nested", "bitnest_greedy_accept",
                  "bitnest_greedy_accept_noalloc", "bitnest_kv_attention", "bitnest_linear_chain",
                  "bitnest_stream_read"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def bitnest_abi_version() -> int:
    return lib().bitnest_abi_version()


def bitnest_status_string(status: int) -> str:
    return lib().bitnest_status_string(int(status)).decode()


def _stream(t: torch.Tensor, *others):
    """torch's current stream of t's device, after checking that every tensor
    of the call is on that device and that it is the current device (the
    library works on the calling thread's current device)."""
    dev = t.device
    for o in others:
        if o is not None and o.device != dev:
            raise ValueError("all tensors of a call must be on one device, got %s and %s" % (dev, o.device))
    if torch.cuda.current_device() != dev.index:
        raise ValueError("the tensors are on %s but the current device is cuda:%d; call under "
                         "torch.cuda.device(%s)" % (dev, torch.cuda.current_device(), dev))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(status: int, what: str):
    if status != OK:
        raise BitnestError(status, what)


def _scale_tensor(scale: torch.Tensor) -> torch.Tensor:
    # fp16 scales may come as float16 or as their int16 bit patterns
    if scale.dtype == torch.float16:
        return scale.view(torch.int16)
    return scale


def bitnest_quant_act(x: torch.Tensor, act_group: int = 0, xq: torch.Tensor | None = None,
                      xs: torch.Tensor | None = None):
    """x fp32 [M, K] -> (xq int8 [M, K], xs fp32 [M] or [M, K/128])."""
    _need(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M,) if act_group == 0 else (M, K // GROUP), dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, (M, K))
    _need(xs, "xs", torch.float32, (M,) if act_group == 0 else (M, K // GROUP))
    _call(lib().bitnest_quant_act(_p(x), M, K, act_group, _p(xq), _p(xs), _stream(x, xq, xs)),
          "bitnest_quant_act")
    return xq, xs


def _linear_shapes(xq, xs, hi, scale, act_group):
    _need(xq, "xq", torch.int8)
    if xq.dim() != 2:
        raise ValueError("xq must be [M, K]")
    M, K = xq.shape
    _need(hi, "hi", torch.uint8)
    if hi.dim() != 2 or hi.shape[1] * 2 != K:
        raise ValueError("hi must be [N, K/2] with K=%d, got %s" % (K, tuple(hi.shape)))
    N = hi.shape[0]
    _need(scale, "scale", torch.int16, (N, K // GROUP))
    _need(xs, "xs", torch.float32, (M,) if act_group == 0 else (M, K // GROUP))
    return M, N, K


def bitnest_linear_draft(xq: torch.Tensor, xs: torch.Tensor, hi: torch.Tensor, scale: torch.Tensor,
                         act_group: int = 0, y: torch.Tensor | None = None) -> torch.Tensor:
    """Draft W4A8 linear: y fp32 [M, N] from the hi plane only."""
    scale = _scale_tensor(scale)
    M, N, K = _linear_shapes(xq, xs, hi, scale, act_group)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _need(y, "y", torch.float32, (M, N))
    _call(lib().bitnest_linear_draft(_p(xq), _p(xs), act_group, _p(hi), _p(scale), _p(y), M, N, K,
                                     _stream(xq, xs, hi, scale, y)), "bitnest_linear_draft")
    return y


def bitnest_linear_target(xq: torch.Tensor, xs: torch.Tensor, hi: torch.Tensor, lo: torch.Tensor,
                          scale: torch.Tensor, act_group: int = 0,
                          y: torch.Tensor | None = None) -> torch.Tensor:
    """Target W8A8 linear: y fp32 [M, N] from the hi and lo planes."""
    scale = _scale_tensor(scale)
    M, N, K = _linear_shapes(xq, xs, hi, scale, act_group)
    _need(lo, "lo", torch.uint8, tuple(hi.shape))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _need(y, "y", torch.float32, (M, N))
    _call(lib().bitnest_linear_target(_p(xq), _p(xs), act_group, _p(hi), _p(lo), _p(scale), _p(y),
                                      M, N, K, _stream(xq, xs, hi, lo, scale, y)), "bitnest_linear_target")
    return y


def bitnest_linear_partials(xq: torch.Tensor, hi: torch.Tensor, lo: torch.Tensor | None = None):
    """Integer partials int32 [M, N, K/128]: P_hi, or (P_hi, P_lo, P8) with ``lo``."""
    _need(xq, "xq", torch.int8)
    M, K = xq.shape
    _need(hi, "hi", torch.uint8)
    if hi.dim() != 2 or hi.shape[1] * 2 != K:
        raise ValueError("hi must be [N, K/2]")
    N = hi.shape[0]
    G = K // GROUP
    p_hi = torch.empty((M, N, G), dtype=torch.int32, device=xq.device)
    p_lo = p8 = None
    if lo is not None:
        _need(lo, "lo", torch.uint8, tuple(hi.shape))
        p_lo = torch.empty_like(p_hi)
        p8 = torch.empty_like(p_hi)
    _call(lib().bitnest_linear_partials(_p(xq), _p(hi), _p(lo), _p(p_hi), _p(p_lo), _p(p8), M, N, K,
                                        _stream(xq, hi, lo, p_hi, p_lo, p8)), "bitnest_linear_partials")
    return p_hi if lo is None else (p_hi, p_lo, p8)


def bitnest_hadamard_quant_act(x: torch.Tensor, block: int, xq: torch.Tensor | None = None,
                               xs: torch.Tensor | None = None, xr: torch.Tensor | None = None,
                               rotated: bool = False):
    """R4 rotation (blocks of ``block`` columns) then per-token quantisation:
    x fp32 [M, K] -> (xq int8 [M, K], xs fp32 [M]), plus the rotated fp32
    [M, K] as a third value when ``rotated`` (or ``xr``) is given."""
    _need(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    if xr is None and rotated:
        xr = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, (M, K))
    _need(xs, "xs", torch.float32, (M,))
    if xr is not None:
        _need(xr, "xr", torch.float32, (M, K))
    _call(lib().bitnest_hadamard_quant_act(_p(x), M, K, int(block), _p(xq), _p(xs), _p(xr), _stream(x, xq, xs, xr)),
          "bitnest_hadamard_quant_act")
    return (xq, xs) if xr is None else (xq, xs, xr)


def _quant_linear(x, hi, lo, scale, act_group, y, xq, xs, what, block=0):
    _need(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    scale = _scale_tensor(scale)
    _need(hi, "hi", torch.uint8)
    if hi.dim() != 2 or hi.shape[1] * 2 != K:
        raise ValueError("hi must be [N, K/2] with K=%d, got %s" % (K, tuple(hi.shape)))
    N = hi.shape[0]
    _need(scale, "scale", torch.int16, (N, K // GROUP))
    if lo is not None:
        _need(lo, "lo", torch.uint8, tuple(hi.shape))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M,) if act_group == 0 else (M, K // GROUP), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (M, N))
    _need(xq, "xq", torch.int8, (M, K))
    _need(xs, "xs", torch.float32, (M,) if act_group == 0 else (M, K // GROUP))
    if block:
        if lo is None:
            st = lib().bitnest_hadamard_quant_linear_draft(_p(x), int(block), _p(hi), _p(scale), _p(y), _p(xq),
                                                           _p(xs), M, N, K, _stream(x, hi, scale, y, xq, xs))
        else:
            st = lib().bitnest_hadamard_quant_linear_target(_p(x), int(block), _p(hi), _p(lo), _p(scale), _p(y),
                                                            _p(xq), _p(xs), M, N, K,
                                                            _stream(x, hi, lo, scale, y, xq, xs))
    elif lo is None:
        st = lib().bitnest_quant_linear_draft(_p(x), act_group, _p(hi), _p(scale), _p(y), _p(xq), _p(xs),
                                              M, N, K, _stream(x, hi, scale, y, xq, xs))
    else:
        st = lib().bitnest_quant_linear_target(_p(x), act_group, _p(hi), _p(lo), _p(scale), _p(y), _p(xq),
                                               _p(xs), M, N, K, _stream(x, hi, lo, scale, y, xq, xs))
    _call(st, what)
    return y, xq, xs


FUSED_MAX_MK = 16384
FUSED_MAX_TOKENS = 4
FUSED_MAX_TOKENS_K = 4096
FUSED_MAX_TOKENS_N = 8192


def fused_in_one_launch(M: int, N: int, K: int, rot_block: int = 0) -> bool:
    """Whether bitnest_quant_linear_* (or, with rot_block, the rotating call)
    runs as a single kernel launch for this shape (otherwise it is a
    quantisation launch followed by the linear); the library's rule: one
    token and K <= 16384, or up to four tokens, K <= 4096 and N <= 8192
    without the rotation."""
    return (M == 1 and K <= FUSED_MAX_MK) or (rot_block == 0 and 1 <= M <= FUSED_MAX_TOKENS
                                              and K <= FUSED_MAX_TOKENS_K and N <= FUSED_MAX_TOKENS_N)


def bitnest_quant_linear_draft(x: torch.Tensor, hi: torch.Tensor, scale: torch.Tensor, act_group: int = 0,
                               y: torch.Tensor | None = None, xq: torch.Tensor | None = None,
                               xs: torch.Tensor | None = None):
    """Quantise x and run the draft linear in one call: returns (y, xq, xs)."""
    return _quant_linear(x, hi, None, scale, act_group, y, xq, xs, "bitnest_quant_linear_draft")


def bitnest_quant_linear_target(x: torch.Tensor, hi: torch.Tensor, lo: torch.Tensor, scale: torch.Tensor,
                                act_group: int = 0, y: torch.Tensor | None = None,
                                xq: torch.Tensor | None = None, xs: torch.Tensor | None = None):
    """Quantise x and run the target linear in one call: returns (y, xq, xs)."""
    return _quant_linear(x, hi, lo, scale, act_group, y, xq, xs, "bitnest_quant_linear_target")


def bitnest_hadamard_quant_linear_draft(x: torch.Tensor, block: int, hi: torch.Tensor, scale: torch.Tensor,
                                        y: torch.Tensor | None = None, xq: torch.Tensor | None = None,
                                        xs: torch.Tensor | None = None):
    """R4 rotation, per-token quantisation and the draft linear in one call: (y, xq, xs)."""
    return _quant_linear(x, hi, None, scale, 0, y, xq, xs, "bitnest_hadamard_quant_linear_draft", block=block)


def bitnest_hadamard_quant_linear_target(x: torch.Tensor, block: int, hi: torch.Tensor, lo: torch.Tensor,
                                         scale: torch.Tensor, y: torch.Tensor | None = None,
                                         xq: torch.Tensor | None = None, xs: torch.Tensor | None = None):
    """R4 rotation, per-token quantisation and the target linear in one call: (y, xq, xs)."""
    return _quant_linear(x, hi, lo, scale, 0, y, xq, xs, "bitnest_hadamard_quant_linear_target", block=block)


def bitnest_pack_nested(W: torch.Tensor, hi: torch.Tensor | None = None, lo: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None):
    """fp32 weights [N, K] -> (hi uint8 [N, K/2], lo uint8 [N, K/2], scale int16 fp16 bits
    [N, K/128]): the nested packing rule of bitnest.h."""
    _need(W, "W", torch.float32)
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    if hi is None:
        hi = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if lo is None:
        lo = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((N, K // GROUP), dtype=torch.int16, device=W.device)
    scale = _scale_tensor(scale)
    _need(hi, "hi", torch.uint8, (N, K // 2))
    _need(lo, "lo", torch.uint8, (N, K // 2))
    _need(scale, "scale", torch.int16, (N, K // GROUP))
    _call(lib().bitnest_pack_nested(_p(W), N, K, _p(hi), _p(lo), _p(scale), _stream(W, hi, lo, scale)),
          "bitnest_pack_nested")
    return hi, lo, scale


def bitnest_greedy_accept_workspace_bytes(R: int, V: int) -> int:
    return int(lib().bitnest_greedy_accept_workspace_bytes(R, V))


def bitnest_greedy_accept(logits: torch.Tensor, draft: torch.Tensor, targ: torch.Tensor | None = None,
                          result: torch.Tensor | None = None, work: torch.Tensor | None = None):
    """Greedy verification: logits fp32 [gamma + 1, V], draft int32 [gamma] ->
    (targ int32 [gamma + 1], result int32 [2] = {accepted count, next token}).
    work: device scratch of bitnest_greedy_accept_workspace_bytes(R, V) bytes
    (allocated here when not given)."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    _need(draft, "draft", torch.int32, (R - 1,))
    if targ is None:
        targ = torch.empty((R,), dtype=torch.int32, device=logits.device)
    if result is None:
        result = torch.empty((2,), dtype=torch.int32, device=logits.device)
    _need(targ, "targ", torch.int32, (R,))
    _need(result, "result", torch.int32, (2,))
    need = bitnest_greedy_accept_workspace_bytes(R, V)
    if work is None:
        work = torch.empty((max(need, 16),), dtype=torch.uint8, device=logits.device)
    _need(work, "work", work.dtype)
    _call(lib().bitnest_greedy_accept(_p(logits), R, V, _p(draft) if R > 1 else None, _p(targ), _p(result),
                                      _p(work), work.numel() * work.element_size(),
                                      _stream(logits, draft, targ, result, work)),
          "bitnest_greedy_accept")
    return targ, result


def bitnest_greedy_accept_noalloc(logits: torch.Tensor, draft: torch.Tensor, targ: torch.Tensor | None = None,
                                  result: torch.Tensor | None = None):
    """bitnest_greedy_accept with the library's per-device scratch instead of
    a workspace: allocates nothing on the device when ``targ`` and ``result``
    are given. Calls that overlap on one device race on that scratch."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    _need(draft, "draft", torch.int32, (R - 1,))
    if targ is None:
        targ = torch.empty((R,), dtype=torch.int32, device=logits.device)
    if result is None:
        result = torch.empty((2,), dtype=torch.int32, device=logits.device)
    _need(targ, "targ", torch.int32, (R,))
    _need(result, "result", torch.int32, (2,))
    _call(lib().bitnest_greedy_accept_noalloc(_p(logits), R, V, _p(draft) if R > 1 else None, _p(targ),
                                              _p(result), _stream(logits, draft, targ, result)),
          "bitnest_greedy_accept_noalloc")
    return targ, result


def bitnest_stream_read(buf: torch.Tensor, sink: torch.Tensor, never: int = 0x5EEDF00D, depth: int = 4,
                        waves_per_cu: int = 0):
    """Read all of ``buf`` (contiguous, 16-byte aligned, a multiple of 1 KiB)
    with the plane stream's loads and no arithmetic: a measurement of the HBM
    read ceiling. ``depth`` items in flight per wave (2, 4 or 8), at most
    ``waves_per_cu`` resident waves per compute unit (0: as many as fit).
    ``sink`` (one int32 on the device) is written only if the folded data
    equal ``never``."""
    _need(buf, "buf", buf.dtype)
    _need(sink, "sink", torch.int32)
    nbytes = buf.numel() * buf.element_size()
    _call(lib().bitnest_stream_read(_p(buf), nbytes, depth, waves_per_cu, never & 0xFFFFFFFF, _p(sink),
                                    _stream(buf, sink)), "bitnest_stream_read")


KV_HEAD_DIM = 128


def kv_pack(kv: torch.Tensor):
    """fp32 K or V entries [Hkv, T, 128] (head-major) -> nested cache planes (hi, lo
    uint8 [Hkv, T, 64], scale int16 fp16 bits [Hkv, T]): bitnest_pack_nested over
    the Hkv T vectors."""
    _need(kv, "kv", torch.float32)
    if kv.dim() != 3 or kv.shape[2] != KV_HEAD_DIM:
        raise ValueError("kv must be [Hkv, T, 128]")
    Hkv, T, _ = kv.shape
    hi, lo, sc = bitnest_pack_nested(kv.reshape(Hkv * T, KV_HEAD_DIM))
    return hi.view(Hkv, T, KV_HEAD_DIM // 2), lo.view(Hkv, T, KV_HEAD_DIM // 2), sc.view(Hkv, T)


def bitnest_kv_attention_workspace_bytes(M: int, Hq: int, T: int) -> int:
    return int(lib().bitnest_kv_attention_workspace_bytes(M, Hq, T))


def bitnest_kv_attention(q: torch.Tensor, k_hi: torch.Tensor, k_scale: torch.Tensor, v_hi: torch.Tensor,
                         v_scale: torch.Tensor, k_lo: torch.Tensor | None = None, v_lo: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, work: torch.Tensor | None = None,
                         T: int | None = None) -> torch.Tensor:
    """Decode attention over the nested KV cache: q fp32 [M, Hq, 128]; head-major
    planes uint8 [Hkv, t_cap, 64]; scales [Hkv, t_cap] (fp16 or their int16 bits);
    the first T positions of each head are read (T defaults to t_cap); KV4
    without the lo planes, KV8 with them. Returns out fp32 [M, Hq, 128]."""
    _need(q, "q", torch.float32)
    if q.dim() != 3 or q.shape[2] != KV_HEAD_DIM:
        raise ValueError("q must be [M, Hq, 128]")
    M, Hq, _ = q.shape
    _need(k_hi, "k_hi", torch.uint8)
    if k_hi.dim() != 3 or k_hi.shape[2] != KV_HEAD_DIM // 2:
        raise ValueError("k_hi must be [Hkv, t_cap, 64]")
    Hkv, t_cap, _ = k_hi.shape
    if T is None:
        T = t_cap
    k_scale, v_scale = _scale_tensor(k_scale), _scale_tensor(v_scale)
    _need(v_hi, "v_hi", torch.uint8, tuple(k_hi.shape))
    _need(k_scale, "k_scale", torch.int16, (Hkv, t_cap))
    _need(v_scale, "v_scale", torch.int16, (Hkv, t_cap))
    if (k_lo is None) != (v_lo is None):
        raise ValueError("give both lo planes or neither")
    if k_lo is not None:
        _need(k_lo, "k_lo", torch.uint8, tuple(k_hi.shape))
        _need(v_lo, "v_lo", torch.uint8, tuple(k_hi.shape))
    if out is None:
        out = torch.empty((M, Hq, KV_HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (M, Hq, KV_HEAD_DIM))
    need = bitnest_kv_attention_workspace_bytes(M, Hq, T)
    if work is None:
        work = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _need(work, "work", work.dtype)
    _call(lib().bitnest_kv_attention(_p(q), M, Hq, Hkv, T, t_cap, _p(k_hi), _p(k_lo), _p(k_scale), _p(v_hi),
                                     _p(v_lo), _p(v_scale), _p(out), _p(work), work.numel() * work.element_size(),
                                     _stream(q, k_hi, k_lo, k_scale, v_hi, v_lo, v_scale, out, work)),
          "bitnest_kv_attention")
    return out


class ChainLink(ctypes.Structure):
    """One link of bitnest_linear_chain (the C struct bitnest_chain_linear)."""
    _fields_ = [("x", ctypes.c_void_p), ("hi", ctypes.c_void_p), ("lo", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("y", ctypes.c_void_p), ("xq", ctypes.c_void_p),
                ("xs", ctypes.c_void_p), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("act_group", ctypes.c_int32), ("rot_block", ctypes.c_int32)]


CHAIN_MAX_M = 4


class LinearChain:
    """A fixed chain of (quantise, linear) steps run by one bitnest_linear_chain
    launch per call of run(). Each link is a dict with the tensors of one
    bitnest_quant_linear_draft/_target call: x fp32 [M, K], hi uint8 [N, K/2],
    lo (target chains; None or absent for draft chains), scale [N, K/128],
    y fp32 [M, N], optional xq int8 [M, K] and xs fp32 [M] or [M, K/128]
    (both or neither), act_group 0 or 128. The link table is built and copied
    to the device once here (so run() can be captured in a HIP graph), and the
    constructor waits until that copy and the workspace's zero fill are done,
    so run() may be called on any stream of the device; the tensors must stay
    alive and in place, which this object ensures by holding them. A link's x
    may be an earlier link's y."""

    def __init__(self, links, max_polls: int = 0, work: torch.Tensor | None = None):
        if not links:
            raise ValueError("a chain needs at least one link")
        self.count = len(links)
        self.M = None
        self.device = None
        self._keep = []
        host = (ChainLink * self.count)()
        for j, d in enumerate(links):
            x, hi, scale, y = d["x"], d["hi"], _scale_tensor(d["scale"]), d["y"]
            lo, xq, xs = d.get("lo"), d.get("xq"), d.get("xs")
            g = int(d.get("act_group", 0))
            _need(x, "x", torch.float32)
            if x.dim() != 2:
                raise ValueError("link %d: x must be [M, K]" % j)
            M, K = x.shape
            if self.M is None:
                self.M, self.device = M, x.device
            elif M != self.M:
                raise ValueError("link %d: every link must have the same M" % j)
            _need(hi, "hi", torch.uint8)
            if hi.dim() != 2 or hi.shape[1] * 2 != K:
                raise ValueError("link %d: hi must be [N, K/2] with K=%d" % (j, K))
            N = hi.shape[0]
            _need(scale, "scale", torch.int16, (N, K // GROUP))
            if lo is not None:
                _need(lo, "lo", torch.uint8, tuple(hi.shape))
            _need(y, "y", torch.float32, (M, N))
            if (xq is None) != (xs is None):
                raise ValueError("link %d: give xq and xs together" % j)
            if xq is not None:
                _need(xq, "xq", torch.int8, (M, K))
                _need(xs, "xs", torch.float32, (M,) if g == 0 else (M, K // GROUP))
            for name, t in (("x", x), ("hi", hi), ("lo", lo), ("scale", scale), ("y", y), ("xq", xq), ("xs", xs)):
                if t is not None and t.device != self.device:
                    raise ValueError("link %d: %s is on %s, the chain runs on %s" % (j, name, t.device, self.device))
            host[j] = ChainLink(x.data_ptr(), hi.data_ptr(), None if lo is None else lo.data_ptr(),
                                scale.data_ptr(), y.data_ptr(), None if xq is None else xq.data_ptr(),
                                None if xs is None else xs.data_ptr(), N, K, g, 0)
            self._keep += [x, hi, lo, scale, y, xq, xs]
        self._host = host
        raw = bytes(memoryview(host).cast("B"))
        self._dev = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)
        nbytes = int(lib().bitnest_chain_workspace_bytes())
        if work is None:
            work = torch.zeros((nbytes,), dtype=torch.uint8, device=self.device)
        _need(work, "work", torch.uint8)
        if work.device != self.device:
            raise ValueError("work is on %s, the chain runs on %s" % (work.device, self.device))
        if work.numel() < nbytes:
            raise ValueError("work must hold %d bytes" % nbytes)
        self.work = work
        self.max_polls = int(max_polls)
        # the link table's copy and the workspace's zero fill were enqueued on
        # the current stream; run() may be called on another one (a capture
        # stream, a worker stream), so they must be complete before it
        torch.cuda.current_stream(self.device).synchronize()

    def run(self):
        """Enqueue the chain on torch's current stream (one launch)."""
        _call(lib().bitnest_linear_chain(ctypes.cast(self._host, ctypes.c_void_p), _p(self._dev), self.count,
                                         self.M, self.max_polls, _p(self.work), self.work.numel(),
                                         _stream(self.work)), "bitnest_linear_chain")

    def timed_out(self) -> bool:
        """Whether a wait of some call on this workspace ran out (synchronises)."""
        return bool(self.work[4:8].view(torch.int32).item())


def bitnest_linear_chain(links, max_polls: int = 0):
    """Build a LinearChain over `links` and run it once; returns the chain."""
    c = LinearChain(links, max_polls=max_polls)
    c.run()
    return c


# Short aliases
quant_act = bitnest_quant_act
linear_draft = bitnest_linear_draft
linear_target = bitnest_linear_target
linear_partials = bitnest_linear_partials
quant_linear_draft = bitnest_quant_linear_draft
quant_linear_target = bitnest_quant_linear_target
hadamard_quant_act = bitnest_hadamard_quant_act
hadamard_quant_linear_draft = bitnest_hadamard_quant_linear_draft
hadamard_quant_linear_target = bitnest_hadamard_quant_linear_target
pack_nested = bitnest_pack_nested
greedy_accept = bitnest_greedy_accept
kv_attention = bitnest_kv_attention
