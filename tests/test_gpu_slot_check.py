"""GPU tests of gdn_check_slots, the device-side debug check of a decode
step's slot preconditions (include/gdn.h), through the binding: each kind of
violation, padding rows, in place and twin, a batch larger than the check's
workgroup, and random slot arrays against the same rules restated here in
plain Python."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_recurrent_decode_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _rules(rd, wr, N):
    """Rows that break a precondition: a slot outside [0, N); a real row (read
    slot not 0) sharing its read slot with another real row; for a twin write,
    a real row writing its own read slot, slot 0, or another row's nonzero
    read or write slot."""
    bad = []
    B = len(rd)
    for r in range(B):
        rs = int(rd[r])
        ws = int(wr[r]) if wr is not None else rs
        b = not (0 <= rs < N and 0 <= ws < N)
        if not b and rs != 0:
            if wr is not None and (ws == rs or ws == 0):
                b = True
            for j in range(B):
                if j == r:
                    continue
                rj = int(rd[j])
                wj = int(wr[j]) if wr is not None else rj
                if rj != 0 and rj == rs:
                    b = True
                if wr is not None and ((rj != 0 and rj == ws) or (wj != 0 and (wj == ws or wj == rs))):
                    b = True
        if b:
            bad.append(r)
    return bad


def _run(gdn, torch, rd, wr, N):
    t = torch
    rdt = t.tensor(np.asarray(rd, np.int32), device="cuda")
    wrt = None if wr is None else t.tensor(np.asarray(wr, np.int32), device="cuda")
    res = gdn.check_slots(rdt, wrt, N=N).cpu().tolist()
    bad = _rules(rd, wr, N)
    assert res == [len(bad), bad[0] if bad else -1], (res, bad)
    return res


def test_valid_twin_and_in_place_with_padding(gdn, torch):
    rd = [3, 0, 5, 7, 0, 9]
    wr = [4, 0, 6, 8, 0, 10]
    assert _run(gdn, torch, rd, wr, N=11) == [0, -1]
    assert _run(gdn, torch, rd, None, N=11) == [0, -1]


@pytest.mark.parametrize("rd,wr,expect", [
    ([3, 5, 7, 11], [4, 6, 8, 2], [1, 3]),            # read slot past N
    ([3, 5, -1, 9], [4, 6, 8, 10], [1, 2]),           # negative read slot
    ([3, 5, 7, 9], [4, 6, 8, 12], [1, 3]),            # write slot past N
    ([3, 5, 7, 9], [4, 5, 8, 10], [1, 1]),            # twin write onto its own read slot
    ([3, 5, 7, 9], [4, 6, 0, 10], [1, 2]),            # twin write into the null slot
    ([3, 5, 7, 5], [4, 6, 8, 10], [2, 1]),            # two real rows share a read slot
    ([3, 5, 7, 9], [4, 9, 8, 10], [2, 1]),            # a write slot is another row's read slot
    ([3, 5, 7, 9], [4, 6, 8, 6], [2, 1]),             # two rows write one slot
    ([0, 5, 0, 9], [4, 6, 4, 10], [0, -1]),           # padding rows: their slots are not used
    ([0, 5, 7, 9], [6, 6, 8, 10], [1, 1]),            # ... but a padding row's write slot is another row's
], ids=["read-past-N", "read-negative", "write-past-N", "write-own-read", "write-null", "shared-read",
        "write-other-read", "shared-write", "padding-rows", "padding-write-clash"])
def test_each_violation(gdn, torch, rd, wr, expect):
    assert _run(gdn, torch, rd, wr, N=11) == expect


def test_in_place_shared_read_slot(gdn, torch):
    assert _run(gdn, torch, [3, 5, 3, 0, 0], None, N=9) == [2, 0]


def test_more_rows_than_the_workgroup(gdn, torch):
    rng = np.random.Generator(np.random.PCG64(5))
    perm = rng.permutation(np.arange(1, 6001)).astype(np.int32)
    rd, wr = perm[:3000].copy(), perm[3000:].copy()
    assert _run(gdn, torch, rd, wr, N=6001) == [0, -1]
    wr[2500] = rd[1700]
    assert _run(gdn, torch, rd, wr, N=6001) == [2, 1700]


def test_random_slot_arrays(gdn, torch):
    rng = np.random.Generator(np.random.PCG64(6))
    for _ in range(40):
        B = int(rng.integers(1, 40))
        N = int(rng.integers(2, 3 * B + 3))
        rd = rng.integers(-1, N + 1, size=B).astype(np.int32)
        rd[rng.random(B) < 0.2] = 0
        twin = bool(rng.integers(0, 2))
        wr = rng.integers(-1, N + 1, size=B).astype(np.int32) if twin else None
        _run(gdn, torch, rd, wr, N)
