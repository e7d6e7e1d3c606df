"""The greedy verification entry point that allocates nothing
(bitnest_greedy_accept_noalloc, the library's per-device scratch) against the
workspace entry point bitnest_greedy_accept, through the C ABI. Outputs are
integers and must be identical; two calls in a row, the second with a
smaller input, so that the second reads the scratch the first left behind."""
import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _case(R, V, seed):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    for r in range(0, R, 2):                       # ties at the maximum of every other row
        cols = rng.choice(V, size=min(V, 4), replace=False)
        logits[r, cols] = logits[r].max() + 1.0
    t = np.argmax(logits, axis=1).astype(np.int32)
    draft = t[:R - 1].copy()
    if R > 2:
        draft[R // 2] = (draft[R // 2] + 1) % V     # a rejection half-way
    return logits, draft


# the largest scratch use (32 rows x 64 slices = 16 KiB), then smaller calls
CALLS = [(32, 300000, 1), (4, 128256, 2), (1, 1000, 3)]


def test_noalloc_matches_workspace_call_in_a_row():
    targ = torch.empty((32,), dtype=torch.int32, device="cuda")
    res = torch.empty((2,), dtype=torch.int32, device="cuda")
    for R, V, seed in CALLS:
        logits, draft = _case(R, V, seed)
        lg, dr = torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda()
        t_ref, r_ref = bn.bitnest_greedy_accept(lg, dr)
        t, r = bn.bitnest_greedy_accept_noalloc(lg, dr, targ[:R], res)
        torch.cuda.synchronize()
        assert torch.equal(t, t_ref), (R, V)
        assert torch.equal(r, r_ref), (R, V)
        t_o, n_o, next_o = oracle.greedy_accept(logits, draft)
        assert np.array_equal(t.cpu().numpy(), t_o)
        assert r.cpu().tolist() == [n_o, next_o]


def test_noalloc_calls_in_one_stream_order_do_not_interfere():
    # two calls queued back to back on one stream (no synchronisation between
    # them): the second overwrites the scratch only after the first is done
    a, da = _case(8, 262147, 4)
    b, db = _case(3, 50000, 5)
    ta, ra = bn.bitnest_greedy_accept_noalloc(torch.from_numpy(a).cuda(), torch.from_numpy(da).cuda())
    tb, rb = bn.bitnest_greedy_accept_noalloc(torch.from_numpy(b).cuda(), torch.from_numpy(db).cuda())
    torch.cuda.synchronize()
    for (lg, dr, t, r) in ((a, da, ta, ra), (b, db, tb, rb)):
        t_o, n_o, next_o = oracle.greedy_accept(lg, dr)
        assert np.array_equal(t.cpu().numpy(), t_o)
        assert r.cpu().tolist() == [n_o, next_o]


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lg = torch.zeros((33, 16), dtype=torch.float32, device="cuda")
    dr = torch.zeros((32,), dtype=torch.int32, device="cuda")
    with pytest.raises(bn.BitnestError) as e:
        bn.bitnest_greedy_accept_noalloc(lg, dr)
    assert e.value.status == bn.EUNSUPPORTED
