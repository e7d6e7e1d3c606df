"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point that include/bitnest.h declares, and rejects bad arguments on the
host, before anything reaches the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

import w8_quantized_linear_amd as bn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnest.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitnest_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("bitnest_quant_act", "bitnest_linear_draft", "bitnest_linear_target",
              "bitnest_linear_partials", "bitnest_status_string", "bitnest_abi_version",
              "bitnest_quant_linear_draft", "bitnest_quant_linear_target", "bitnest_hadamard_quant_act",
              "bitnest_hadamard_quant_linear_draft", "bitnest_hadamard_quant_linear_target",
              "bitnest_pack_nested", "bitnest_greedy_accept", "bitnest_kv_attention",
              "bitnest_kv_attention_workspace_bytes", "bitnest_greedy_accept_workspace_bytes",
              "bitnest_greedy_accept_noalloc", "bitnest_stream_read"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bn.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", bn.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(L, name)
    # C linkage: no mangled bitnest_ symbols leak out
    assert not [s for s in exported if s.startswith("_Z") and "bitnest_" in s and not s.startswith("_ZN7bitnest")]


def test_version_and_status_strings():
    assert bn.bitnest_abi_version() == 8
    seen = set()
    for s in range(5):
        txt = bn.bitnest_status_string(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert bn.bitnest_status_string(99) == "unknown status"
    assert bn.bitnest_status_string(0) == "ok"


# Fake, 16-byte-aligned, non-null addresses: validation must reject every call
# below before dereferencing anything or calling HIP.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
D = ctypes.c_void_p(0x40000)
E = ctypes.c_void_p(0x50000)
F = ctypes.c_void_p(0x60000)
MIS = ctypes.c_void_p(0x10004)
NUL = None


def _q(x, M, K, g, xq, xs):
    return bn.lib().bitnest_quant_act(x, M, K, g, xq, xs, None)


def _d(xq, xs, g, hi, sc, y, M, N, K):
    return bn.lib().bitnest_linear_draft(xq, xs, g, hi, sc, y, M, N, K, None)


def _t(xq, xs, g, hi, lo, sc, y, M, N, K):
    return bn.lib().bitnest_linear_target(xq, xs, g, hi, lo, sc, y, M, N, K, None)


def _p(xq, hi, lo, ph, pl, p8, M, N, K):
    return bn.lib().bitnest_linear_partials(xq, hi, lo, ph, pl, p8, M, N, K, None)


def _kv(q, M, Hq, Hkv, T, kh, kl, ks, vh, vl, vs, out, w, wb, t_cap=None):
    return bn.lib().bitnest_kv_attention(q, M, Hq, Hkv, T, T if t_cap is None else t_cap, kh, kl, ks, vh, vl, vs,
                                         out, w, wb, None)


_DEFAULT = object()


def _ga(lg, R, V, dr, tg, res, w=_DEFAULT, wb=1 << 20):
    return bn.lib().bitnest_greedy_accept(lg, R, V, dr, tg, res, A if w is _DEFAULT else w, wb, None)


def _gn(lg, R, V, dr, tg, res):
    return bn.lib().bitnest_greedy_accept_noalloc(lg, R, V, dr, tg, res, None)


def _sr(p, nbytes, sink, depth=4, wpc=0):
    return bn.lib().bitnest_stream_read(p, nbytes, depth, wpc, 0, sink, None)


def _pk(W, N, K, hi, lo, sc):
    return bn.lib().bitnest_pack_nested(W, N, K, hi, lo, sc, None)


def _h(x, M, K, b, xq, xs, xr):
    return bn.lib().bitnest_hadamard_quant_act(x, M, K, b, xq, xs, xr, None)


def _hd(x, b, hi, sc, y, xq, xs, M, N, K):
    return bn.lib().bitnest_hadamard_quant_linear_draft(x, b, hi, sc, y, xq, xs, M, N, K, None)


def _ht(x, b, hi, lo, sc, y, xq, xs, M, N, K):
    return bn.lib().bitnest_hadamard_quant_linear_target(x, b, hi, lo, sc, y, xq, xs, M, N, K, None)


@pytest.mark.parametrize("call,status", [
    # quant_act
    (lambda: _q(NUL, 1, 128, 0, B, C), bn.EINVAL),
    (lambda: _q(A, 1, 128, 0, NUL, C), bn.EINVAL),
    (lambda: _q(A, 1, 128, 0, B, NUL), bn.EINVAL),
    (lambda: _q(A, 1, 128, 64, B, C), bn.EINVAL),
    (lambda: _q(A, -1, 128, 0, B, C), bn.EINVAL),
    (lambda: _q(A, 1, 0, 0, B, C), bn.EINVAL),
    (lambda: _q(A, 1, 100, 0, B, C), bn.EINVAL),
    (lambda: _q(A, 1, 16384 + 128, 0, B, C), bn.EUNSUPPORTED),
    (lambda: _q(MIS, 1, 128, 0, B, C), bn.EALIGN),
    (lambda: _q(A, 1, 128, 0, MIS, C), bn.EALIGN),
    (lambda: _q(A, 1, 128, 128, B, MIS), bn.EALIGN),
    (lambda: _q(A, 0, 128, 0, B, C), bn.OK),                # empty: nothing launched
    # draft
    (lambda: _d(NUL, B, 0, C, D, E, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, NUL, 0, C, D, E, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, NUL, D, E, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, C, NUL, E, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, NUL, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 7, C, D, E, 1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, E, -1, 8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, E, 1, -8, 128), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, E, 1, 8, 0), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, E, 1, 8, 192), bn.EINVAL),
    (lambda: _d(A, B, 0, C, D, E, 33, 8, 128), bn.EUNSUPPORTED),
    (lambda: _d(A, B, 0, C, D, E, 1, 8, 16512), bn.EUNSUPPORTED),
    (lambda: _d(MIS, B, 0, C, D, E, 1, 8, 128), bn.EALIGN),
    (lambda: _d(A, B, 0, MIS, D, E, 1, 8, 128), bn.EALIGN),
    (lambda: _d(A, B, 0, C, MIS, E, 1, 8, 128), bn.EALIGN),
    (lambda: _d(A, B, 0, C, D, MIS, 1, 8, 128), bn.EALIGN),
    (lambda: _d(A, B, 0, C, D, E, 0, 8, 128), bn.OK),
    (lambda: _d(A, B, 0, C, D, E, 4, 0, 128), bn.OK),
    # target
    (lambda: _t(A, B, 0, C, NUL, D, E, 1, 8, 128), bn.EINVAL),
    (lambda: _t(A, B, 0, C, MIS, D, E, 1, 8, 128), bn.EALIGN),
    (lambda: _t(A, B, 128, C, F, D, E, 1, 8, 100), bn.EINVAL),
    (lambda: _t(A, B, 0, C, F, D, E, 40, 8, 128), bn.EUNSUPPORTED),
    (lambda: _t(A, B, 0, C, F, D, E, 0, 8, 128), bn.OK),
    (lambda: _t(A, B, 0, C, F, D, E, 1, 300000, 16384), bn.EUNSUPPORTED),   # plane > 2 GiB
    # partials
    (lambda: _p(NUL, B, C, D, E, F, 1, 8, 128), bn.EINVAL),
    (lambda: _p(A, NUL, C, D, E, F, 1, 8, 128), bn.EINVAL),
    (lambda: _p(A, B, C, NUL, E, F, 1, 8, 128), bn.EINVAL),
    (lambda: _p(A, B, C, D, NUL, F, 1, 8, 128), bn.EINVAL),
    (lambda: _p(A, B, C, D, E, NUL, 1, 8, 128), bn.EINVAL),
    (lambda: _p(A, B, NUL, D, NUL, NUL, 1, 8, 130), bn.EINVAL),
    (lambda: _p(A, B, C, D, E, MIS, 1, 8, 128), bn.EALIGN),
    (lambda: _p(A, B, NUL, D, NUL, NUL, 0, 8, 128), bn.OK),
    # empty calls accept NULL pointers (torch's empty tensors have none)
    (lambda: _q(NUL, 0, 128, 0, NUL, NUL), bn.OK),
    (lambda: _d(NUL, NUL, 0, NUL, NUL, NUL, 0, 8, 128), bn.OK),
    (lambda: _t(NUL, NUL, 0, NUL, NUL, NUL, NUL, 3, 0, 128), bn.OK),
    (lambda: _p(NUL, NUL, NUL, NUL, NUL, NUL, 0, 0, 128), bn.OK),
    (lambda: _d(NUL, NUL, 0, NUL, NUL, NUL, 0, 8, 100), bn.EINVAL),
    # R4 rotation + quantisation: block a power of two in [2, 512] dividing K
    (lambda: _h(A, 1, 512, 0, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 1, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 96, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 1024, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 384, 256, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 100, 4, B, C, NUL), bn.EINVAL),
    (lambda: _h(NUL, 1, 512, 512, B, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 512, NUL, C, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 512, B, NUL, NUL), bn.EINVAL),
    (lambda: _h(A, 1, 512, 512, B, C, MIS), bn.EALIGN),
    (lambda: _h(MIS, 1, 512, 512, B, C, NUL), bn.EALIGN),
    (lambda: _h(A, 1, 16384 + 512, 512, B, C, NUL), bn.EUNSUPPORTED),
    (lambda: _h(NUL, 0, 512, 512, NUL, NUL, NUL), bn.OK),
    (lambda: _hd(A, 0, B, C, D, E, F, 1, 8, 512), bn.EINVAL),
    (lambda: _hd(A, 3, B, C, D, E, F, 1, 8, 512), bn.EINVAL),
    (lambda: _hd(A, 512, B, C, D, E, F, 1, 8, 640), bn.EINVAL),
    (lambda: _hd(A, 512, NUL, C, D, E, F, 1, 8, 512), bn.EINVAL),
    (lambda: _hd(A, 512, B, C, D, E, F, 33, 8, 512), bn.EUNSUPPORTED),
    (lambda: _hd(NUL, 512, NUL, NUL, NUL, NUL, NUL, 0, 8, 512), bn.OK),
    (lambda: _ht(A, 512, B, NUL, C, D, E, F, 1, 8, 512), bn.EINVAL),
    (lambda: _ht(A, 512, B, MIS, C, D, E, F, 1, 8, 512), bn.EALIGN),
    # read-ceiling measurement: whole KiB, at least one, below 4 GiB
    (lambda: _sr(NUL, 1024, B), bn.EINVAL),
    (lambda: _sr(A, 1024, NUL), bn.EINVAL),
    (lambda: _sr(A, 0, B), bn.EINVAL),
    (lambda: _sr(A, 1000, B), bn.EINVAL),
    (lambda: _sr(A, 1 << 32, B), bn.EINVAL),
    (lambda: _sr(MIS, 1024, B), bn.EALIGN),
    (lambda: _sr(A, 1024, B, 3), bn.EINVAL),
    (lambda: _sr(A, 1024, B, 16), bn.EINVAL),
    (lambda: _sr(A, 1024, B, 4, -1), bn.EINVAL),
    # nested packing
    (lambda: _pk(NUL, 4, 128, B, C, D), bn.EINVAL),
    (lambda: _pk(A, 4, 128, NUL, C, D), bn.EINVAL),
    (lambda: _pk(A, 4, 128, B, NUL, D), bn.EINVAL),
    (lambda: _pk(A, 4, 128, B, C, NUL), bn.EINVAL),
    (lambda: _pk(A, -1, 128, B, C, D), bn.EINVAL),
    (lambda: _pk(A, 4, 100, B, C, D), bn.EINVAL),
    (lambda: _pk(A, 4, 128, B, C, MIS), bn.EALIGN),
    (lambda: _pk(MIS, 4, 128, B, C, D), bn.EALIGN),
    (lambda: _pk(A, 300000, 16384, B, C, D), bn.EUNSUPPORTED),
    (lambda: _pk(NUL, 0, 128, NUL, NUL, NUL), bn.OK),
    # greedy verification
    (lambda: _ga(A, 0, 100, B, C, D), bn.EINVAL),
    (lambda: _ga(A, 4, 0, B, C, D), bn.EINVAL),
    (lambda: _ga(A, 33, 100, B, C, D), bn.EUNSUPPORTED),
    (lambda: _ga(A, 4, (1 << 30) + 1, B, C, D), bn.EUNSUPPORTED),
    (lambda: _ga(A, 4, 2 ** 31 - 1, B, C, D), bn.EUNSUPPORTED),
    (lambda: _ga(NUL, 4, 100, B, C, D), bn.EINVAL),
    (lambda: _ga(A, 4, 100, NUL, C, D), bn.EINVAL),
    (lambda: _ga(A, 4, 100, B, NUL, D), bn.EINVAL),
    (lambda: _ga(A, 4, 100, B, C, NUL), bn.EINVAL),
    (lambda: _ga(MIS, 4, 100, B, C, D), bn.EALIGN),
    (lambda: _ga(A, 4, 100, B, C, MIS), bn.EALIGN),
    (lambda: _ga(A, 4, 100, B, C, D, NUL), bn.EINVAL),
    (lambda: _ga(A, 4, 100, B, C, D, A, 31), bn.EINVAL),
    (lambda: _ga(A, 4, 100, B, C, D, MIS), bn.EALIGN),
    # greedy verification without a workspace (the library's scratch)
    (lambda: _gn(A, 0, 100, B, C, D), bn.EINVAL),
    (lambda: _gn(A, 4, 0, B, C, D), bn.EINVAL),
    (lambda: _gn(A, 33, 100, B, C, D), bn.EUNSUPPORTED),
    (lambda: _gn(A, 4, (1 << 30) + 1, B, C, D), bn.EUNSUPPORTED),
    (lambda: _gn(NUL, 4, 100, B, C, D), bn.EINVAL),
    (lambda: _gn(A, 4, 100, NUL, C, D), bn.EINVAL),
    (lambda: _gn(A, 4, 100, B, NUL, D), bn.EINVAL),
    (lambda: _gn(A, 4, 100, B, C, NUL), bn.EINVAL),
    (lambda: _gn(MIS, 4, 100, B, C, D), bn.EALIGN),
    (lambda: _gn(A, 4, 100, B, C, MIS), bn.EALIGN),
    # nested KV attention: every case fails validation (none may launch)
    (lambda: _kv(A, 0, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 4, 30, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 4, 32, 8, 3, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 8, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EUNSUPPORTED),
    # T 64 = 2^31 bytes of one head: beyond the offset range
    (lambda: _kv(A, 1, 32, 8, 1 << 25, B, NUL, C, D, NUL, E, F, A, 1 << 40), bn.EUNSUPPORTED),
    # fewer positions allocated per head than the sequence holds
    (lambda: _kv(A, 4, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20, 99), bn.EINVAL),
    (lambda: _kv(A, 1, 65536, 65536, 4, B, NUL, C, D, NUL, E, F, A, 1 << 40), bn.EUNSUPPORTED),
    # M * (Hq / Hkv) = 2^32: beyond the row limit (not wrapped to 0)
    (lambda: _kv(A, 1 << 20, 1 << 12, 1, 1 << 20, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EUNSUPPORTED),
    (lambda: _kv(NUL, 4, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 4, 32, 8, 100, B, NUL, C, D, NUL, E, F, NUL, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 4, 32, 8, 100, B, C, C, D, NUL, E, F, A, 1 << 20), bn.EINVAL),
    (lambda: _kv(A, 4, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1000), bn.EINVAL),
    (lambda: _kv(MIS, 4, 32, 8, 100, B, NUL, C, D, NUL, E, F, A, 1 << 20), bn.EALIGN),
    (lambda: _kv(A, 4, 32, 8, 100, B, NUL, C, D, NUL, E, MIS, A, 1 << 20), bn.EALIGN),
])
def test_host_validation(call, status):
    assert call() == status
def test_kv_workspace_size():
    # at most one split per 64-position chunk and at most 512 splits, each
    # with (M Hq) rows x (128 values + maximum + sum) floats
    assert bn.bitnest_kv_attention_workspace_bytes(4, 32, 100) == 2 * 4 * 32 * 130 * 4
    assert bn.bitnest_kv_attention_workspace_bytes(1, 32, 2048) == 32 * 32 * 130 * 4
    assert bn.bitnest_kv_attention_workspace_bytes(1, 32, 64 * 512) == 512 * 32 * 130 * 4
    assert bn.bitnest_kv_attention_workspace_bytes(4, 32, 131072) == 512 * 4 * 32 * 130 * 4
    assert bn.bitnest_kv_attention_workspace_bytes(0, 32, 10) == 0
    # the largest T: still 512 splits (no overflow in the chunk count)
    assert bn.bitnest_kv_attention_workspace_bytes(1, 32, 2 ** 31 - 1) == 512 * 32 * 130 * 4


def test_accept_workspace_size():
    # one (value, index) pair of 8 bytes per row and slice of about 4096
    # logits, from 1 to 64 slices
    assert bn.bitnest_greedy_accept_workspace_bytes(4, 128256) == 4 * 32 * 8
    assert bn.bitnest_greedy_accept_workspace_bytes(1, 1) == 8
    assert bn.bitnest_greedy_accept_workspace_bytes(32, 4097) == 32 * 2 * 8
    assert bn.bitnest_greedy_accept_workspace_bytes(2, 10 ** 6) == 2 * 64 * 8
    assert bn.bitnest_greedy_accept_workspace_bytes(0, 100) == 0
    # the largest V: still 64 slices; beyond it (or beyond the row limit) no size
    assert bn.bitnest_greedy_accept_workspace_bytes(2, 2 ** 30) == 2 * 64 * 8
    assert bn.bitnest_greedy_accept_workspace_bytes(2, 2 ** 30 + 1) == 0
    assert bn.bitnest_greedy_accept_workspace_bytes(33, 100) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((1, 128), dtype=torch.float32)
    with pytest.raises(ValueError):
        bn.bitnest_quant_act(x)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # no fallback: without the built HIP library every call path raises
    monkeypatch.setattr(bn, "_lib", None)
    monkeypatch.setattr(bn, "library_path", str(tmp_path / "libbitnest.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bn.lib()
    with pytest.raises(RuntimeError, match="not built"):
        bn.bitnest_abi_version()


def test_smoke_refuses_to_run_without_a_gpu():
    import torch
    import __graft_entry__
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(RuntimeError, match="needs a GPU"):
        __graft_entry__.smoke()
