"""The top-k select at row lengths no workload reaches (one wave per row up to
4096 keys, one workgroup per row beyond, up to the 8192 limit), on seeded
score rows with many exact ties and both signed zeros: the lists must equal
the oracle's rank rule bit for bit."""
import numpy as np
import pytest

import oracle
from tests import gpu_support as gs
from workloads.inputs import score_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,sparsity", [(3000, 0.95), (4096, 0.9), (5000, 0.9), (8192, 0.5)])
def test_select_long_rows_match_oracle(n, sparsity):
    import torch
    from block_sparse_video_map_amd import vsa
    # one head, n single-row video tiles, no prefix
    prob = vsa.Problem(1, 1, 64, (1, 1, 64 * n), (), ((1, 1, 64),), "bf16")
    sz = vsa.vsa_query_sizes(prob, sparsity)
    assert sz.max_video_tiles == n
    k = sz.k[0]
    assert k == oracle.keep_count(sparsity, n)
    gs.log(f"[select] n={n} k={k}")
    host = score_rows(4400 + n, n, n)
    scores = torch.from_numpy(host).cuda().reshape(-1)
    kv = torch.full((sz.idx_elems,), -9, dtype=torch.int32, device="cuda")
    vsa.vsa_select_topk(prob, scores, sparsity, kv)
    torch.cuda.synchronize()
    got = kv.view(n, sz.k_max).cpu().numpy()
    rows = np.random.default_rng(n).choice(n, size=96, replace=False)
    rows = np.unique(np.concatenate([rows, [0, 1, n - 2, n - 1]]))
    want = oracle.select_topk(host[rows], k)
    np.testing.assert_array_equal(got[rows, :k], want)
    assert (got[rows, k:] == -1).all()
