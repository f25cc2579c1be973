"""dv_check_indices on crafted lists (GPU): each rule a list can break is reported on its own
row, valid lists report 0, and the flags match a plain host scan of the same lists."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def host_flags(lists, n):
    """The same rules, scanned on the host entry by entry."""
    out = []
    for row in lists:
        f = 0
        for j, v in enumerate(row):
            if v < 0 or v >= n:
                f |= 1
            if j > 0 and v < row[j - 1]:
                f |= 2
            if j > 0 and v == row[j - 1]:
                f |= 4
        out.append(f)
    return np.array(out, np.int32)


def run(dv, lists, n):
    idx = torch.from_numpy(np.ascontiguousarray(lists, np.int32)).cuda()
    status = torch.full((idx.shape[0],), -1, dtype=torch.int32, device="cuda")
    dv.dv_check_indices(idx, n, status)
    torch.cuda.synchronize()
    return status.cpu().numpy()


def test_crafted_rows(dv):
    n = 50
    rows = [
        [0, 3, 7, 49],       # valid
        [0, 3, 3, 49],       # repeat
        [0, 7, 3, 49],       # out of order
        [0, 3, 7, 50],       # beyond n
        [-1, 3, 7, 49],      # negative
        [5, 5, 2, 60],       # all three
        [49, 48, 47, 46],    # descending
    ]
    got = run(dv, rows, n)
    expect = [0, dv.DV_IDX_DUPLICATE, dv.DV_IDX_ORDER, dv.DV_IDX_RANGE, dv.DV_IDX_RANGE,
              dv.DV_IDX_RANGE | dv.DV_IDX_ORDER | dv.DV_IDX_DUPLICATE, dv.DV_IDX_ORDER]
    assert got.tolist() == expect
    assert np.array_equal(got, host_flags(rows, n))


@pytest.mark.parametrize("k", [1, 255, 256, 257, 2458, 49152])
def test_long_rows_one_fault_each(dv, k):
    """Rows longer than one block's sweep: a single bad entry anywhere (first, last, across a
    sweep boundary) is found; the valid rows (sorted draws, and the full identity list) report 0."""
    n = 49152
    rng = np.random.default_rng(k)
    base = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
    rows = [base.copy()]
    if k == n:
        rows.append(np.arange(n, dtype=np.int32))
    if k >= 2:
        for pos in sorted({1, k // 2, 256 % k if k > 256 else 1, k - 1}):
            r = base.copy(); r[pos] = r[pos - 1]; rows.append(r)            # repeat
            r = base.copy(); r[pos - 1], r[pos] = r[pos], r[pos - 1]; rows.append(r)   # swap
    r = base.copy(); r[-1] = n; rows.append(r)                              # beyond n at the end
    r = base.copy(); r[0] = -5; rows.append(r)                              # negative at the start
    got = run(dv, np.stack(rows), n)
    assert np.array_equal(got, host_flags([list(map(int, r)) for r in rows], n))
    assert got[0] == 0 and (k != n or got[1] == 0)


def test_topk_output_is_valid(dv):
    """dv_topk's lists pass the check (the form every gather expects)."""
    scores = torch.randn(3, 49152, device="cuda")
    idx = torch.empty(3, 2458, dtype=torch.int32, device="cuda")
    dv.dv_topk(scores, 2458, idx)
    status = torch.full((3,), -1, dtype=torch.int32, device="cuda")
    dv.dv_check_indices(idx, 49152, status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 0, 0]


def test_empty_lists(dv):
    status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    dv.dv_check_indices(None, 10, status, k=0)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 0, 0, 0]
