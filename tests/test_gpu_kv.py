"""GPU parity of decode attention over the nested KV cache (draft KV4, target
KV8) against the CPU oracle, through the C ABI.

The caches are packed on the CPU by the oracle (in its [T, Hkv] order) and
uploaded in the library's head-major layout, so every input of the oracle is
its own. Bar, per (token, query head): max over the 128 dimensions of
|out - out_oracle| <= 1e-5 * max|out_oracle| of that (token, head), plus
1e-8 * max|V| so that an output that cancels to nearly zero is not held to
a bound below fp32 resolution (the oracle is fp64; the kernel accumulates
in fp32 over splits of 64-position chunks with a running softmax, then
merges the splits; measured on these cases: at most 7e-7 of the output's
own magnitude). At long contexts a flat softmax makes the output about
max|V| / sqrt(T), so a bar relative to max|V| alone would admit
percent-level errors there; this one does not. Invariants checked bit for bit on the GPU: KV8 with lo
planes of 8 equals KV4; token i of an M-token call equals a one-token call on
the cache cut after its last visible position.
"""
import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn

pytestmark = pytest.mark.gpu

TOL = 1e-5          # relative to each (token, head) output
FLOOR = 1e-8        # relative to max|V|


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _cache(T, Hkv, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    out = []
    for scale in (spread, 1.0):
        X = (rng.standard_normal((T, Hkv, 128)) * scale * rng.uniform(0.3, 2.0, size=(T, Hkv, 1))).astype(np.float32)
        hi, lo, sc = oracle.pack_nested(X.reshape(T * Hkv, 128))
        out.append((hi.reshape(T, Hkv, 64), lo.reshape(T, Hkv, 64), sc.reshape(T, Hkv)))
    return out          # (K planes, V planes)


def _head_major(a, t_cap, fill):
    # [T, Hkv, ...] (the oracle's layout) -> the cache's [Hkv, t_cap, ...]:
    # positions past T hold `fill`, which the kernel must not read
    T = a.shape[0]
    out = np.full((a.shape[1], t_cap) + a.shape[2:], fill, dtype=a.dtype)
    out[:, :T] = np.swapaxes(a, 0, 1)
    return out


def _run(q, kc, vc, kv8, t_cap=None):
    T = kc[0].shape[0]
    t_cap = T if t_cap is None else t_cap
    # past T: codes 0xFF and a huge scale (fp16 60000), so a read past the
    # sequence would show
    d = lambda a, fill: torch.from_numpy(np.ascontiguousarray(_head_major(a, t_cap, fill))).cuda()
    big = np.uint16(0x7B53)
    out = bn.bitnest_kv_attention(torch.from_numpy(np.ascontiguousarray(q)).cuda(),
                                  d(kc[0], 0xFF), d(kc[2], big).view(torch.int16), d(vc[0], 0xFF),
                                  d(vc[2], big).view(torch.int16),
                                  d(kc[1], 0xFF) if kv8 else None, d(vc[1], 0xFF) if kv8 else None, T=T)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(q, kc, vc, kv8):
    return oracle.kv_attention(q, kc[0], kc[2], vc[0], vc[2], kc[1] if kv8 else None, vc[1] if kv8 else None)


def _check(got, want, vmax):
    err = np.abs(got - want).max(axis=-1)             # [M, Hq]
    bound = TOL * np.abs(want).max(axis=-1) + FLOOR * vmax
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert (err <= bound).all(), ("token, head", worst, err[worst], bound[worst])


def _vmax(vc, kv8):
    hi, lo, sc = vc
    T, Hkv, _ = hi.shape
    V = oracle.dequant(hi.reshape(T * Hkv, 64), sc.reshape(T * Hkv, 1), lo.reshape(T * Hkv, 64) if kv8 else None)
    return np.abs(V).max()


@pytest.mark.parametrize("M,Hq,Hkv,T", [
    (1, 32, 8, 2048), (4, 32, 8, 2048), (4, 32, 8, 100), (4, 32, 8, 4), (1, 8, 8, 1), (2, 16, 2, 300),
    (3, 12, 4, 257), (1, 32, 8, 8192), (4, 32, 8, 64), (4, 32, 8, 65), (1, 4, 1, 129),
    # long contexts: several 64-position chunks per split, ragged tails, and
    # (one KV head) hundreds of splits up to the 512 cap
    (1, 32, 8, 32768), (4, 32, 8, 20001), (1, 4, 1, 40000), (2, 8, 1, 32768), (4, 16, 16, 12345),
])
@pytest.mark.parametrize("kv8", [False, True])
def test_kv_attention_matches_oracle(M, Hq, Hkv, T, kv8):
    kc, vc = _cache(T, Hkv, seed=M * 1000 + T, spread=0.5)
    q = np.random.default_rng(T).standard_normal((M, Hq, 128)).astype(np.float32)
    got = _run(q, kc, vc, kv8)
    want = _ref(q, kc, vc, kv8)
    _check(got, want, _vmax(vc, kv8))


@pytest.mark.parametrize("M,T,t_cap", [(1, 2048, 2049), (4, 1000, 4096), (4, 20001, 20480)])
@pytest.mark.parametrize("kv8", [False, True])
def test_kv_attention_reads_only_the_first_t_positions_of_each_head(M, T, t_cap, kv8):
    # the cache holds t_cap positions per head; those past T are filled with
    # codes and scales that would dominate the result if they were read
    kc, vc = _cache(T, 8, seed=T + t_cap)
    q = np.random.default_rng(T).standard_normal((M, 32, 128)).astype(np.float32)
    got = _run(q, kc, vc, kv8, t_cap=t_cap)
    want = _ref(q, kc, vc, kv8)
    _check(got, want, _vmax(vc, kv8))


@pytest.mark.parametrize("kv8", [False, True])
def test_kv_attention_head_bases_beyond_2_31(kv8):
    # t_cap so large that heads 4..7 start more than 2^31 bytes into their
    # planes (head h at h * t_cap * 64 bytes); only the first T positions of
    # each head are read. The cache is built on the GPU; positions past T
    # hold codes and scales that would dominate the result if read.
    M, Hq, Hkv, T = 4, 32, 8, 3000
    t_cap = (1 << 31) // (64 * 4) + 1000
    assert 4 * t_cap * 64 > 2**31 - 1 and T * 64 < 2**31
    kc, vc = _cache(T, Hkv, seed=77)
    q = np.random.default_rng(77).standard_normal((M, Hq, 128)).astype(np.float32)

    def d(a, fill, dtype):
        out = torch.full((Hkv, t_cap) + a.shape[2:], fill, dtype=dtype, device="cuda")
        out[:, :T] = torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1)).view(dtype_np[dtype])).cuda()
        return out

    dtype_np = {torch.uint8: np.uint8, torch.int16: np.int16}
    big = 0x7B53                    # fp16 60000 (its bit pattern fits int16)
    out = bn.bitnest_kv_attention(torch.from_numpy(q).cuda(),
                                  d(kc[0], 0xFF, torch.uint8), d(kc[2], big, torch.int16),
                                  d(vc[0], 0xFF, torch.uint8), d(vc[2], big, torch.int16),
                                  d(kc[1], 0xFF, torch.uint8) if kv8 else None,
                                  d(vc[1], 0xFF, torch.uint8) if kv8 else None, T=T)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    torch.cuda.empty_cache()
    _check(got, _ref(q, kc, vc, kv8), _vmax(vc, kv8))


def test_kv_peaked_scores():
    # large scores (sharp softmax) stay accurate
    kc, vc = _cache(512, 8, seed=7, spread=3.0)
    q = (np.random.default_rng(8).standard_normal((4, 32, 128)) * 3).astype(np.float32)
    got = _run(q, kc, vc, True)
    want = _ref(q, kc, vc, True)
    _check(got, want, _vmax(vc, True))


@pytest.mark.parametrize("T", [300, 20000])    # one chunk per split / runs of chunks
def test_kv8_with_lo_8_equals_kv4_on_gpu(T):
    kc, vc = _cache(T, 8, seed=9)
    q = np.random.default_rng(9).standard_normal((4, 32, 128)).astype(np.float32)
    k8 = (kc[0], np.full_like(kc[1], 0x88), kc[2])
    v8 = (vc[0], np.full_like(vc[1], 0x88), vc[2])
    a = _run(q, k8, v8, True)
    b = _run(q, kc, vc, False)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("T", [200, 9000])
def test_kv_token_rows_equal_one_token_calls_on_the_cut_cache(T):
    M = 4
    kc, vc = _cache(T, 8, seed=10)
    q = np.random.default_rng(10).standard_normal((M, 32, 128)).astype(np.float32)
    full = _run(q, kc, vc, True)
    for i in range(M):
        n = T - M + i + 1
        cut_k = tuple(np.ascontiguousarray(a[:n]) for a in kc)
        cut_v = tuple(np.ascontiguousarray(a[:n]) for a in vc)
        one = _run(q[i:i + 1], cut_k, cut_v, True)
        assert np.array_equal(full[i].view(np.uint32), one[0].view(np.uint32))


def test_kv_pack_writes_the_oracle_planes():
    # the cache write path (bitnest_pack_nested over the Hkv T vectors of a
    # head-major cache)
    rng = np.random.default_rng(11)
    X = rng.standard_normal((8, 33, 128)).astype(np.float32)
    hi, lo, sc = bn.kv_pack(torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    h_r, l_r, s_r = oracle.pack_nested(X.reshape(8 * 33, 128))
    assert hi.shape == (8, 33, 64) and sc.shape == (8, 33)
    assert np.array_equal(hi.cpu().numpy().reshape(8 * 33, 64), h_r)
    assert np.array_equal(lo.cpu().numpy().reshape(8 * 33, 64), l_r)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16).reshape(8 * 33, 1), s_r)


def test_kv_sequence_longer_than_the_cache_is_rejected():
    # T > t_cap: rejected on the host before any launch
    kc, vc = _cache(64, 8, seed=12)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(_head_major(a, 64, 0))).cuda()
    q = torch.zeros((1, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(bn.BitnestError) as e:
        bn.bitnest_kv_attention(q, d(kc[0]), d(kc[2]).view(torch.int16), d(vc[0]), d(vc[2]).view(torch.int16), T=65)
    assert e.value.status == bn.EINVAL
