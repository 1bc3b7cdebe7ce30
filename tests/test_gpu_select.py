"""The GPU top-B select, bit-exact against the oracle's select on identical
fp32 score vectors (the library's select entry point, through the C ABI)."""

import numpy as np
import pytest

from oracle import select_top_b

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402


def _cases():
    rng = np.random.default_rng(2024)
    yield "random", rng.random(4352).astype(np.float32), 4096
    yield "random_small_b", rng.random(4352).astype(np.float32) * 7, 1
    yield "b_is_pool_minus_1", rng.random(1280).astype(np.float32), 1279
    yield "pool_le_b", rng.random(300).astype(np.float32), 1024
    yield "all_equal", np.full(2304, 0.25, dtype=np.float32), 2048
    yield "all_zero", np.zeros(777, dtype=np.float32), 100
    q = (rng.integers(0, 5, 4352) / 4).astype(np.float32)
    yield "quantised_ties", q, 4096
    yield "quantised_ties_mid", q, 2000
    # realistic scores: sums of probabilities, heavy-tailed, many near-ties
    s = (rng.pareto(3.0, 4352) * 0.3).astype(np.float32)
    s[rng.choice(4352, 500, replace=False)] = s[0]
    yield "pareto_with_ties", s, 4096
    yield "denormals_and_zero", np.array([0.0, 1e-45, 2e-45, 1e-38, 0.0, 3.0],
                                         dtype=np.float32), 3
    yield "large_pool", rng.random(32768).astype(np.float32), 30000
    yield "one", np.array([5.0], dtype=np.float32), 1


@pytest.mark.parametrize("name,scores,budget", list(_cases()), ids=[c[0] for c in _cases()])
def test_select_bit_exact(name, scores, budget):
    d = torch.from_numpy(scores).cuda()
    got = skv.select_topb(d, budget).cpu().numpy()
    ref = select_top_b(scores, np.arange(scores.shape[0]), budget)
    np.testing.assert_array_equal(got, ref)


def test_select_many_random_budgets():
    rng = np.random.default_rng(7)
    for trial in range(50):
        n = int(rng.integers(1, 6000))
        b = int(rng.integers(1, n + 50))
        s = (rng.integers(0, 1 + int(rng.integers(1, 300)), n) / 7).astype(np.float32)
        got = skv.select_topb(torch.from_numpy(s).cuda(), b).cpu().numpy()
        np.testing.assert_array_equal(got, select_top_b(s, np.arange(n), b), err_msg=str(trial))
