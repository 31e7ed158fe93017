"""The allocation-free top-k (indexer_topk_noalloc), called through the C ABI, against
indexer_topk with a caller workspace: two calls in a row on long rows (the second smaller
than the first, so it runs on the scratch array's leftovers), one with the decode scorer's
row histogram, and a short-row call. Selections must be identical (same logits, exact
selection), and the oracle's full sort agrees on the first call's rows."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ifp4():
    import sparse_attention_indexer_fp4_amd as m

    return m


def _logits(rows, ld, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((rows, ld), generator=g, dtype=torch.float32) * 30.0 + 200.0
    x[:, ::97] = x[:, 5:6]  # ties across the row
    return x.to(dev())


def _with_ws(ifp4, lg, rl, max_len, k, hist=None):
    out = torch.full((lg.shape[0], k), -7, dtype=torch.int32, device=dev())
    ws = torch.zeros(max(ifp4.indexer_topk_workspace_bytes(lg.shape[0], max_len, k), 16), dtype=torch.uint8,
                     device=dev())
    ifp4.indexer_topk(lg, rl, max_len, k, out, ws, hist)
    return out


def _no_alloc(ifp4, lg, rl, max_len, k, hist=None):
    out = torch.full((lg.shape[0], k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk_noalloc(lg, rl, max_len, k, out, hist)
    return out


def test_noalloc_matches_workspace_topk(ifp4):
    k = 2048
    # call 1: 16 rows of up to 131072 keys (8.7 MB of scratch), ragged lengths
    rows, ld = 16, 131072
    assert ifp4.indexer_topk_workspace_bytes(rows, ld, k) <= ifp4.NOALLOC_SCRATCH_BYTES
    lg = _logits(rows, ld, 1)
    lens = np.array([131072, 100000, 20000, 2048, 2049, 131071, 65536, 17000] * 2, np.int32)
    rl = torch.from_numpy(lens).to(dev())
    a = _no_alloc(ifp4, lg, rl, ld, k)
    b = _with_ws(ifp4, lg, rl, ld, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ah = a.cpu().numpy()
    s = lg.cpu().numpy().astype(np.float64)
    o = oracle.topk(s[:4], lens[:4], k)  # the oracle's full sort of the same fp32 values
    for r in range(4):
        assert set(ah[r][ah[r] >= 0].tolist()) == set(o[r][o[r] >= 0].tolist())
    # call 2: smaller (3 rows of up to 40000 keys), on what call 1 left in the array
    rows2, ld2 = 3, 40000
    lg2 = _logits(rows2, ld2, 2)
    rl2 = torch.tensor([40000, 39999, 16385], dtype=torch.int32, device=dev())
    a2 = _no_alloc(ifp4, lg2, rl2, ld2, k)
    b2 = _with_ws(ifp4, lg2, rl2, ld2, k)
    torch.cuda.synchronize()
    assert torch.equal(a2, b2)


def test_noalloc_with_scorer_histogram_and_short_rows(ifp4):
    import workloads as W
    from helpers import gpu_decode

    k = 2048
    case = W.decode_case([131072, 70000, 9000], heads=64, topk=k, seed=5)
    g = gpu_decode(case, run_topk=False, fused=True)  # scorer fills the first histogram
    ld = g["ld"]
    hist = g["row_hist"]
    hist_copy = hist.clone()
    a = _no_alloc(ifp4, g["logits"], g["row_len"], ld, k, hist)
    torch.cuda.synchronize()
    assert int(hist.abs().sum().item()) == 0  # left zeroed, as indexer_topk leaves it
    b = _with_ws(ifp4, g["logits"], g["row_len"], ld, k, hist_copy)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # rows short enough for one workgroup each: no scratch involved, same result
    lg = _logits(5, 3000, 3)
    rl = torch.tensor([3000, 10, 2048, 2049, 0], dtype=torch.int32, device=dev())
    assert torch.equal(_no_alloc(ifp4, lg, rl, 3000, 256), _with_ws(ifp4, lg, rl, 3000, 256))
