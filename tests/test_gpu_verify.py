"""GPU parity of moe_verify_accept (acceptance of a verify pass) against the
oracle: kept tokens and their count bit for bit."""

import numpy as np
import pytest

import oracle
from helpers import host, say

pytestmark = pytest.mark.gpu


def _run(logits, draft):
    import torch
    import routed_expert_ffn_gemv_amd as moe
    T, V = logits.shape
    lg = torch.as_tensor(logits, device="cuda")
    dr = torch.as_tensor(np.asarray(draft, np.int32), device="cuda") if T > 1 else None
    out = torch.full((T,), -5, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.moe_verify_workspace_size(T, V), 256), dtype=torch.uint8,
                     device="cuda")
    moe.moe_verify_accept(lg, T, V, dr, out, n, ws)
    torch.cuda.synchronize()
    k = int(host(n)[0])
    return host(out)[:k]


def _greedy(logits):
    return oracle.verify_accept(logits, np.zeros(max(logits.shape[0] - 1, 0), np.int32) - 1)


@pytest.mark.parametrize("kept", [0, 1, 2, 3])
def test_vocabulary_rows(kept):
    """4 rows over a 151,936-entry vocabulary; the first `kept` drafts are
    the model's tokens, the next one is not."""
    rng = np.random.default_rng(10 + kept)
    T, V = 4, 151936
    logits = rng.standard_normal((T, V)).astype(np.float32)
    g = [int(np.argmax(r)) for r in logits]
    draft = np.array([g[i] if i < kept else (g[i] + 1) % V for i in range(T - 1)], np.int32)
    say(f"[gpu] verify accept V={V} kept={kept}")
    got = _run(logits, draft)
    want = oracle.verify_accept(logits, draft)
    np.testing.assert_array_equal(got, want)
    assert len(got) == kept + 1


def test_ties_signed_zeros_and_small_rows():
    T, V = 5, 3000
    logits = np.full((T, V), -1.0, np.float32)
    logits[0, [2999, 17, 1500]] = 4.0            # equal maxima: the lowest index wins
    logits[1, :] = -0.0
    logits[1, 700] = 0.0                         # -0.0 equals +0.0: index 0 wins
    logits[2, [5, 4]] = np.float32(1e-30)
    logits[3, V - 1] = 2.0                       # the last entry
    logits[4, 0] = np.inf
    g = [17, 0, 4, V - 1, 0]
    np.testing.assert_array_equal(_run(logits, np.array(g[:4], np.int32)), g)
    np.testing.assert_array_equal(_run(logits, np.array([17, 0, 5, 1], np.int32)), g[:3])
    for V in (1, 2, 7):
        lg = np.random.default_rng(V).standard_normal((3, V)).astype(np.float32)
        d = np.array([0, 0], np.int32)
        np.testing.assert_array_equal(_run(lg, d), oracle.verify_accept(lg, d))


def test_one_row_and_sixteen_rows():
    rng = np.random.default_rng(3)
    one = rng.standard_normal((1, 50000)).astype(np.float32)
    np.testing.assert_array_equal(_run(one, None), [int(np.argmax(one[0]))])
    lg = rng.standard_normal((16, 32000)).astype(np.float32)
    g = np.argmax(lg, axis=1).astype(np.int32)
    np.testing.assert_array_equal(_run(lg, g[:15]), g)
