"""GPU parity of greedy verification (target argmax per verify row, accepted
prefix, next token) against the CPU oracle, through the C ABI: all outputs
are integers and must match exactly, ties included."""
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


def _case(R, V, seed, ties):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    if ties == "top":
        for r in range(R):
            cols = rng.choice(V, size=min(V, 5), replace=False)
            logits[r, cols] = logits[r].max() + 1.0
    elif ties == "flat":
        logits = np.round(logits).astype(np.float32)        # many equal values
    elif ties == "negative":
        logits = -np.abs(logits) - 5.0
    t = np.argmax(logits, axis=1).astype(np.int32)
    draft = t[:R - 1].copy()
    if R > 1:
        k = int(rng.integers(0, R))                          # R - 1 means: all accepted
        if k < R - 1:
            draft[k] = (draft[k] + 1) % V
    return logits, draft.astype(np.int32)


@pytest.mark.parametrize("R", [1, 2, 4, 8, 32])
@pytest.mark.parametrize("V", [1, 3, 1000, 4096, 4097, 128256, 32001, 262147, 300000])
@pytest.mark.parametrize("ties", ["none", "top", "flat", "negative"])
def test_greedy_accept_exact(R, V, ties):
    logits, draft = _case(R, V, seed=R * 131 + V, ties=ties)
    targ, res = bn.bitnest_greedy_accept(torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda())
    torch.cuda.synchronize()
    t_ref, n_ref, next_ref = oracle.greedy_accept(logits, draft)
    assert np.array_equal(targ.cpu().numpy(), t_ref)
    assert res.cpu().numpy().tolist() == [n_ref, next_ref]


def test_greedy_accept_every_prefix_length():
    R, V = 4, 128256
    logits, _ = _case(R, V, seed=5, ties="top")
    t = np.argmax(logits, axis=1).astype(np.int32)
    lg = torch.from_numpy(logits).cuda()
    for n in range(R):
        draft = t[:R - 1].copy()
        if n < R - 1:
            draft[n] = (draft[n] + 7) % V
        _, res = bn.bitnest_greedy_accept(lg, torch.from_numpy(draft).cuda())
        torch.cuda.synchronize()
        assert res.cpu().numpy().tolist() == [n, int(t[n])]
