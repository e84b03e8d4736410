"""The no-allocation top-k (csa_topk_noalloc, for callers that cannot
allocate) against csa_topk with a caller workspace, through the C ABI: index
sets are integer work, so the two must agree bit for bit.  Two calls in a row
share the library's static scratch, the second on a smaller input; rows short
enough to need no scratch and rows that need all of it are both covered."""
import numpy as np
import pytest
import torch

from tests.gpu_util import progress

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_06_amd as csa
    csa.lib()


def _scores(seed, R, N):
    """Gaussian scores with planted ties, ragged visibility and a -inf tail."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((R, N)).astype(np.float32)
    dup = rng.integers(0, N, size=(R, N // 5))
    s[np.arange(R)[:, None], dup] = s[np.arange(R)[:, None], np.roll(dup, 1, axis=1)]   # ties
    n_valid = rng.integers(N // 2, N + 1, size=R).astype(np.int32)
    n_valid[0] = N
    for r in range(R):
        s[r, n_valid[r]:] = -np.inf
    return torch.from_numpy(s).cuda(), torch.from_numpy(n_valid).cuda()


@pytest.mark.parametrize("cases", [
    [(32, 262144, 1024), (4, 40000, 512)],     # the whole scratch, then a smaller call
    [(8, 300000, 512), (3, 20000, 37), (8, 16384, 512)],
])
def test_topk_noalloc_matches_topk(cases):
    import compressed_sparse_attention_06_amd as csa
    for call, (R, N, k) in enumerate(cases):
        progress(f"topk_noalloc call {call}: R={R} N={N} k={k}")
        scores, n_valid = _scores(1000 + call + N, R, N)
        want = torch.empty((R, k), dtype=torch.int32, device="cuda")
        csa.csa_topk(scores, n_valid, k, want)
        got = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
        csa.csa_topk_noalloc(scores, n_valid, k, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {call}: csa_topk_noalloc differs from csa_topk"
        # and the workspace-less call did use the scratch when the rows are long
        assert (csa.csa_topk_workspace_size(R, N, k) > 0) == (N > 16384)


def test_topk_noalloc_rejects_beyond_scratch():
    import compressed_sparse_attention_06_amd as csa
    scores, n_valid = _scores(7, 2, 1000)
    idx = torch.empty((64, 1024), dtype=torch.int32, device="cuda")
    big = torch.empty((64, 262144), dtype=torch.float32, device="cuda")
    with pytest.raises(csa.CsaError, match="workspace"):
        csa.csa_topk_noalloc(big, None, 1024, idx)
