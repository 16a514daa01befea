"""GPU parity of the device-side join (ja_djoin_*, through the C ABI): the
tuple list and the CSR segments built on the device from split points held
in device memory, bit-exact against the oracle's enumeration
(`oracle.tuple_records`) and, at sizes the oracle cannot enumerate, against
properties that fix the list (every record kept by the predicate, strictly
increasing in group-by order, the closed-form count) plus the host join."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    from tensor_relational_join_amd import device

    return device


def _eq(n, q):
    base, extra = divmod(n, q)
    p = [0]
    for i in range(q):
        p.append(p[-1] + base + (i < extra))
    return p


def _splits_dev(letters, splits):
    import torch

    return torch.tensor([x for c in letters for x in splits[c]], dtype=torch.int64, device="cuda")


def _djoin(dev, einsum, op, splits, params=""):
    import torch

    dj = dev.DeviceJoin(einsum, op, {c: len(v) - 1 for c, v in splits.items()},
                        {c: v[-1] for c, v in splits.items()}, params)
    try:
        dj.run(_splits_dev(dj.letters, splits))
        torch.cuda.synchronize()
        return (dj.letters,) + dj.result()
    finally:
        dj.close()


CASES = [
    ("ij,jk->ik", "contract", {"i": _eq(64, 2), "j": _eq(64, 2), "k": _eq(64, 2)}, "", "ik", None),
    ("ij,kj->ik", "contract", {"i": [0, 3, 10], "j": [0, 1, 5, 7], "k": [0, 4, 9]}, "", "ik", None),
    ("bij,bjk->bik", "contract", {"b": [0, 1, 3], "i": _eq(40, 3), "j": _eq(50, 5), "k": _eq(30, 2)}, "", "bik",
     None),
    ("ij,j->i", "contract", {"i": _eq(100, 7), "j": _eq(90, 9)}, "", "i", None),
    ("bd,df->bf", "contract", {"b": _eq(2048, 2), "d": _eq(4096, 4), "f": _eq(11008, 4)}, "", "bf", None),
    ("bhsd,bhtd,bhtd->bhsd", "attention",
     {"b": [0, 2], "h": [0, 1, 3], "s": [0, 50, 130, 300], "t": [0, 100, 128, 300], "d": [0, 128]},
     "causal=s,t", "bhsd", ("s", "t")),
    ("bhsd,bhtd,bhtd->bhsd", "attention",
     {"b": _eq(2, 2), "h": _eq(4, 4), "s": _eq(2048, 16), "t": _eq(2048, 16), "d": [0, 128]},
     "causal=s,t", "bhsd", ("s", "t")),
    ("bgrsd,bgtd,bgtd->bgrsd", "attention",
     {"b": [0, 1], "g": _eq(8, 8), "r": [0, 4], "s": _eq(8192, 64), "t": _eq(8192, 64), "d": [0, 128]},
     "causal=s,t", "bgrs", ("s", "t")),
    ("bgrsd,bgtd,bgtd->bgrsd", "attention",
     {"b": [0, 2], "g": [0, 1, 3], "r": [0, 1, 2], "s": [0, 70, 200], "t": [0, 130, 200], "d": [0, 128]},
     "", "bgrs", None),
    ("rd,d->rd", "rmsnorm", {"r": _eq(8192, 3), "d": _eq(4096, 8)}, "eps=1e-6", "r", None),
    ("rf,rf->rf", "swiglu", {"r": _eq(8192, 5), "f": _eq(11008, 8)}, "", "rf", None),
    ("rd,rd->rd", "add", {"r": [0, 1], "d": [0, 1]}, "", "rd", None),
]


@pytest.mark.parametrize("einsum,op,splits,params,group_by,causal", CASES)
def test_device_join_matches_oracle(dev, orc, einsum, op, splits, params, group_by, causal):
    letters, rec, seg, status = _djoin(dev, einsum, op, splits, params)
    assert status == 0
    o_rec, o_seg = orc.tuple_records(list(letters), splits, group_by=list(group_by), causal=causal)
    assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg)


PACKED = [
    ({"b": [0, 2], "h": [0, 1, 2], "s": [0, 1024, 2560, 4096], "t": [0, 1024, 2560, 4096], "d": [0, 128]},
     [1024, 2560, 4096], True),
    ({"b": [0, 1], "h": [0, 2], "s": [0, 1024, 4096], "t": [0, 1024, 4096], "d": [0, 128]},
     [1024, 2560, 4096], True),
    ({"b": [0, 1], "h": [0, 1], "s": [0, 700, 3000], "t": [0, 700, 1900, 3000], "d": [0, 128]},
     [700, 1900, 3000], False),
]


@pytest.mark.parametrize("splits,ends,causal", PACKED)
def test_device_join_packed_matches_oracle(dev, orc, splits, ends, causal):
    params = "packed=" + ",".join(map(str, ends)) + (";causal=s,t" if causal else "")
    letters, rec, seg, status = _djoin(dev, "bhsd,bhtd,bhtd->bhsd", "attention", splits, params)
    assert status == 0
    o_rec, o_seg = orc.tuple_records(list(letters), splits, group_by=list("bhsd"),
                                     causal=("s", "t") if causal else None, packed=("s", "t", ends))
    assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg)


def test_device_join_split_points_from_device_data(dev, orc):
    """Which sequence ends the decomposition cuts s and t at is drawn on the
    GPU, and the split points are assembled there and handed to the join
    without a host copy.  Two runs in a row with different cuts reuse one
    handle."""
    import torch

    nseq, T = 24, 6000
    params = "packed=%s;causal=s,t" % ",".join(str(T * (i + 1) // nseq) for i in range(nseq))
    ends = [T * (i + 1) // nseq for i in range(nseq)]
    dj = dev.DeviceJoin("bhsd,bhtd,bhtd->bhsd", "attention", {"b": 1, "h": 4, "s": 9, "t": 9, "d": 1},
                        {"b": 2, "h": 8, "s": T, "t": T, "d": 128}, params)
    try:
        ends_dev = torch.tensor(ends, dtype=torch.int64, device="cuda")
        for seed in (1, 2):
            g = torch.Generator(device="cuda").manual_seed(seed)
            pick = torch.randperm(nseq - 1, generator=g, device="cuda")[:8].sort().values
            cuts = torch.cat([torch.zeros(1, dtype=torch.int64, device="cuda"), ends_dev[pick],
                              ends_dev[-1:]])
            fixed = lambda lo, hi: torch.tensor([lo, hi], dtype=torch.int64, device="cuda")  # noqa: E731
            # letter order b, h, s, d, t
            h_sp = torch.tensor(_eq(8, 4), dtype=torch.int64, device="cuda")
            sp = torch.cat([fixed(0, 2), h_sp, cuts, fixed(0, 128), cuts])
            dj.run(sp)
            rec, seg, status = dj.result()
            assert status == 0
            c = cuts.cpu().tolist()
            splits = {"b": [0, 2], "h": _eq(8, 4), "s": c, "t": c, "d": [0, 128]}
            o_rec, o_seg = orc.tuple_records(list(dj.letters), splits, group_by=list("bhsd"), causal=("s", "t"),
                                             packed=("s", "t", ends))
            assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg)
    finally:
        dj.close()


def test_device_join_rejects_bad_split_points(dev):
    """Split points that are not a tiling, or packed cuts away from a
    sequence end, give a status word and an empty list (never garbage)."""
    import torch

    dj = dev.DeviceJoin("ij,jk->ik", "contract", {"i": 2, "j": 2, "k": 2}, {"i": 10, "j": 10, "k": 10})
    try:
        for bad in ([0, 5, 10, 0, 5, 10, 0, 5, 9],       # k does not end at its extent
                    [0, 5, 10, 0, 10, 10, 0, 5, 10],     # j does not rise strictly
                    [1, 5, 10, 0, 5, 10, 0, 5, 10]):     # i does not start at 0
            dj.run(torch.tensor(bad, dtype=torch.int64, device="cuda"))
            rec, seg, status = dj.result()
            assert status == 1 and rec.shape[0] == 0 and seg.tolist() == [0]
        dj.run(torch.tensor([0, 5, 10, 0, 3, 10, 0, 6, 10], dtype=torch.int64, device="cuda"))
        rec, seg, status = dj.result()
        assert status == 0 and rec.shape[0] == 8 and seg.tolist() == [0, 2, 4, 6, 8]
    finally:
        dj.close()
    dj = dev.DeviceJoin("bhsd,bhtd,bhtd->bhsd", "attention", {"b": 1, "h": 1, "s": 2, "t": 2, "d": 1},
                        {"b": 1, "h": 1, "s": 4096, "t": 4096, "d": 128}, "packed=1024,2560,4096")
    try:
        # letter order b, h, s, d, t; s cut at 2,000 (not a sequence end)
        dj.run(torch.tensor([0, 1, 0, 1, 0, 2000, 4096, 0, 128, 0, 1024, 4096], dtype=torch.int64, device="cuda"))
        rec, seg, status = dj.result()
        assert status == 2 and rec.shape[0] == 0
        dj.run(torch.tensor([0, 1, 0, 1, 0, 2560, 4096, 0, 128, 0, 1024, 4096], dtype=torch.int64, device="cuda"))
        rec, seg, status = dj.result()
        assert status == 0 and rec[:, [2, 4]].tolist() == [[0, 0], [0, 1], [1, 1]]
    finally:
        dj.close()


def _host_join(B, einsum, op, splits, params):
    s = B.ja_spec_create(einsum, op, params)
    try:
        letters = B.ja_spec_letters(s)
        d = B.ja_decomp_create(s, [splits[c][-1] for c in letters], [len(splits[c]) - 1 for c in letters],
                               [splits[c] for c in letters])
        try:
            t = B.ja_join(s, d)
            try:
                return B.ja_tuples_export(t)
            finally:
                B.ja_tuples_destroy(t)
        finally:
            B.ja_decomp_destroy(d)
    finally:
        B.ja_spec_destroy(s)


def test_device_join_long_context_grid(dev):
    """A 131,072-token causal grid (1,024 query and key blocks of 128) over 8
    heads: 8.4 M cells, 4.2 M kept tuples, too many for the oracle's
    enumeration.  Checked by properties that fix the list -- every record
    satisfies the predicate, records rise strictly in group-by order (so none
    repeats and the order is right), the count is the closed form n(n+1)/2
    per head (so none is missing), segments cut exactly where the group-by key
    changes -- and against the host join."""
    from tensor_relational_join_amd import binding as B

    n, H = 1024, 8
    splits = {"b": [0, 1], "h": _eq(H, H), "s": _eq(n * 128, n), "t": _eq(n * 128, n), "d": [0, 128]}
    letters, rec, seg, status = _djoin(dev, "bhsd,bhtd,bhtd->bhsd", "attention", splits, "causal=s,t")
    assert status == 0 and letters == "bhsdt"
    assert rec.shape == (H * n * (n + 1) // 2, 5)
    b, h, s, d, t = (rec[:, i].astype(np.int64) for i in range(5))
    assert (b == 0).all() and (d == 0).all() and (t <= s).all()
    key = (h * n + s) * n + t  # group-by order (b, h, s, d), then t
    assert (np.diff(key) > 0).all()
    gk = h * n + s
    starts = np.flatnonzero(np.diff(gk)) + 1
    assert np.array_equal(seg, np.concatenate([[0], starts, [rec.shape[0]]]))
    h_rec, h_seg = _host_join(B, "bhsd,bhtd,bhtd->bhsd", "attention", splits, "causal=s,t")
    assert np.array_equal(rec, h_rec) and np.array_equal(seg, h_seg)
