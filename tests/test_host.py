"""Host logic of libja checked without a GPU: tuple lists (bit-exact against
the oracle's independent enumeration), relation layout, spec and
decomposition validation, error codes, repartition atom counts, and plan
construction for every configuration."""
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def B():
    from tensor_relational_join_amd import binding

    return binding


def _tuples(B, einsum, op, splits, params=""):
    s = B.ja_spec_create(einsum, op, params)
    try:
        letters = B.ja_spec_letters(s)
        d = B.ja_decomp_create(s, [splits[c][-1] for c in letters], [len(splits[c]) - 1 for c in letters],
                               [splits[c] for c in letters])
        try:
            t = B.ja_join(s, d)
            try:
                rec, seg = B.ja_tuples_export(t)
            finally:
                B.ja_tuples_destroy(t)
        finally:
            B.ja_decomp_destroy(d)
    finally:
        B.ja_spec_destroy(s)
    return letters, rec, seg


def _eq(n, q):
    base, extra = divmod(n, q)
    p = [0]
    for i in range(q):
        p.append(p[-1] + base + (i < extra))
    return p


CASES = [
    ("ij,jk->ik", "contract", {"i": _eq(64, 2), "j": _eq(64, 2), "k": _eq(64, 2)}, "", "ik", None),
    ("bd,df->bf", "contract", {"b": _eq(2048, 2), "d": _eq(4096, 4), "f": _eq(11008, 4)}, "", "bf", None),
    ("bhsd,bhtd,bhtd->bhsd", "attention",
     {"b": _eq(4, 4), "h": _eq(32, 32), "s": _eq(2048, 16), "t": _eq(2048, 16), "d": [0, 128]},
     "causal=s,t", "bhsd", ("s", "t")),
    ("rd,d->rd", "rmsnorm", {"r": _eq(8192, 1), "d": _eq(4096, 8)}, "eps=1e-6", "r", None),
    ("rf,rf->rf", "swiglu", {"r": _eq(8192, 1), "f": _eq(11008, 8)}, "", "rf", None),
    ("td,dn->tn", "contract", {"t": _eq(8192, 2), "d": _eq(4096, 2), "n": _eq(12288, 2)}, "", "tn", None),
    ("ij,kj->ik", "contract", {"i": [0, 3, 10], "j": [0, 1, 5, 7], "k": [0, 4, 9]}, "", "ik", None),
    ("bhsd,bhtd,bhtd->bhsd", "attention",
     {"b": [0, 2], "h": [0, 1, 3], "s": [0, 50, 130, 300], "t": [0, 100, 128, 300], "d": [0, 128]},
     "causal=s,t", "bhsd", ("s", "t")),
    # grouped-query attention (section 3.3): 8 key-value heads of 4 query heads each, 8K tokens
    ("bgrsd,bgtd,bgtd->bgrsd", "attention",
     {"b": [0, 1], "g": _eq(8, 8), "r": [0, 4], "s": _eq(8192, 64), "t": _eq(8192, 64), "d": [0, 128]},
     "causal=s,t", "bgrs", ("s", "t")),
    ("bgrsd,bgtd,bgtd->bgrsd", "attention",
     {"b": [0, 2], "g": [0, 1, 3], "r": [0, 1, 2], "s": [0, 70, 200], "t": [0, 130, 200], "d": [0, 128]},
     "", "bgrs", None),
]


PACKED_CASES = [
    # the pages' section 3.3 example: sequences ending at 1,024, 2,560 and 4,096, cut at every end
    ({"b": [0, 2], "h": [0, 1, 2], "s": [0, 1024, 2560, 4096], "t": [0, 1024, 2560, 4096], "d": [0, 128]},
     [1024, 2560, 4096], True),
    # cut at one end only: the second block holds two sequences
    ({"b": [0, 1], "h": [0, 2], "s": [0, 1024, 4096], "t": [0, 1024, 4096], "d": [0, 128]},
     [1024, 2560, 4096], True),
    # different cuts on the query and key letters, not causal
    ({"b": [0, 1], "h": [0, 1], "s": [0, 700, 3000], "t": [0, 700, 1900, 3000], "d": [0, 128]},
     [700, 1900, 3000], False),
]


@pytest.mark.parametrize("splits,ends,causal", PACKED_CASES)
def test_packed_tuple_lists_match_oracle(B, orc, splits, ends, causal):
    params = "packed=" + ",".join(map(str, ends)) + (";causal=s,t" if causal else "")
    letters, rec, seg = _tuples(B, "bhsd,bhtd,bhtd->bhsd", "attention", splits, params)
    o_rec, o_seg = orc.tuple_records(list(letters), splits, group_by=list("bhsd"),
                                     causal=("s", "t") if causal else None, packed=("s", "t", ends))
    assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg)


def test_packed_sequence_split_points(B):
    """A sequence letter may be split only at sequence ends, and must span
    every sequence (the pages' section 3.3)."""
    s = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "packed=1024,2560,4096;causal=s,t")
    try:
        ok = B.ja_decomp_create(s, [1, 1, 4096, 128, 4096], [1, 1, 2, 1, 3],
                                [[0, 1], [0, 1], [0, 2560, 4096], [0, 128], [0, 1024, 2560, 4096]])
        B.ja_decomp_destroy(ok)
        for sp, ext in (([0, 2048, 4096], 4096), ([0, 1024, 3000], 3000)):
            with pytest.raises(B.JaError) as e:
                B.ja_decomp_create(s, [1, 1, ext, 128, ext], [1, 1, len(sp) - 1, 1, len(sp) - 1],
                                   [[0, 1], [0, 1], sp, [0, 128], sp])
            assert e.value.name == "JA_ERR_DECOMP"
    finally:
        B.ja_spec_destroy(s)
    for bad in ("packed=0,10", "packed=10,5", "packed=", "packed=4,x"):
        with pytest.raises(B.JaError) as e:
            B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", bad)
        assert e.value.name == "JA_ERR_SPEC"
    with pytest.raises(B.JaError):
        B.ja_spec_create("ij,jk->ik", "contract", "packed=4")


@pytest.mark.parametrize("einsum,op,splits,params,group,causal", CASES)
def test_tuple_lists_match_oracle(B, orc, einsum, op, splits, params, group, causal):
    letters, rec, seg = _tuples(B, einsum, op, splits, params)
    o_rec, o_seg = orc.tuple_records(list(letters), splits, group_by=list(group), causal=causal)
    assert rec.dtype == np.int32
    assert np.array_equal(rec, o_rec)
    assert np.array_equal(seg, o_seg)


def test_config_counts(B):
    _, rec, seg = _tuples(B, *CASES[0][:4])
    assert (len(rec), len(seg) - 1) == (8, 4)
    _, rec, seg = _tuples(B, *CASES[1][:4])
    assert (len(rec), len(seg) - 1) == (32, 8)
    _, rec, seg = _tuples(B, *CASES[2][:4])
    assert (len(rec), len(seg) - 1) == (17408, 2048)
    _, rec, seg = _tuples(B, *CASES[5][:4])
    assert (len(rec), len(seg) - 1) == (8, 4)


def test_examples_3_8_3_9_through_the_join(B):
    g = json.load(open(os.path.join(GOLDEN, "example_3_8_3_9_matmul_specs.json")))
    for case in g["cases"]:
        letters, rec, seg = _tuples(B, "ij,jk->ik", "contract", case["splits"])
        assert len(rec) == case["n_specs"]
        assert list(np.diff(seg)) == case["segment_sizes"]
        # boxes of each tuple's projections
        sp = case["splits"]
        for r, want in zip(rec.tolist(), case["specs"]):
            iv = {c: (sp[c][r[letters.index(c)]], sp[c][r[letters.index(c)] + 1]) for c in "ijk"}
            assert [[iv["i"][0], iv["j"][0]], [iv["i"][1], iv["j"][1]]] == want["A"]
            assert [[iv["j"][0], iv["k"][0]], [iv["j"][1], iv["k"][1]]] == want["B"]
            assert [[iv["i"][0], iv["k"][0]], [iv["i"][1], iv["k"][1]]] == want["C"]


def test_relation_layout_matches_oracle(B, orc):
    shape, splits = (7, 10, 3), [[0, 2, 7], [0, 4, 5, 10], [0, 3]]
    rel = B.Relation(shape, splits=splits, dtype=B.JA_F32)
    assert B.ja_relation_bytes(rel) == 7 * 10 * 3 * 4
    assert B.ja_relation_nblocks(rel) == 6
    o = orc.Relation(shape, splits)
    flat = o.pack(np.arange(np.prod(shape)).reshape(shape))
    off = 0
    for key in itertools.product(range(2), range(3), range(1)):
        lo, hi, boff = B.ja_relation_block(rel, key)
        assert (lo, hi) == o.box(key)
        assert boff == off * 4
        # the first element of the block in the oracle's packing is the cell at lo
        assert flat[off] == np.ravel_multi_index(lo, shape)
        off += orc.box_cells((lo, hi))
    # near-equal default splits
    r2 = B.Relation((10,), nblk=(3,), dtype=B.JA_BF16)
    assert [B.ja_relation_block(r2, (k,))[0][0] for k in range(3)] == [0, 4, 7]


@pytest.mark.parametrize("einsum,op,params,code", [
    ("ij,jk", "contract", "", "JA_ERR_SPEC"),
    ("ij,jk->ik", "conv", "", "JA_ERR_SPEC"),
    ("ii,jk->ik", "contract", "", "JA_ERR_SPEC"),
    ("ij,jk->iz", "contract", "", "JA_ERR_SPEC"),
    ("ij,kl->ik", "contract", "", "JA_ERR_SPEC"),          # j and l appear once
    ("bhsd,bhtd,bhtd->bhsd", "attention", "causal=t,s", "JA_ERR_SPEC"),
    ("bhsd,bhtd->bhsd", "attention", "", "JA_ERR_SPEC"),
    ("rd,d->rd", "rmsnorm", "eps=-1", "JA_ERR_SPEC"),
    ("rd,d->rd", "rmsnorm", "bogus=1", "JA_ERR_SPEC"),
    ("ij,jk->ik", "contract", "causal=i,k", "JA_ERR_SPEC"),
    # the attention kernel takes the running maximum on raw scores: the scale must be positive
    ("bhsd,bhtd,bhtd->bhsd", "attention", "scale=0", "JA_ERR_SPEC"),
    ("bhsd,bhtd,bhtd->bhsd", "attention", "scale=-0.5;causal=s,t", "JA_ERR_SPEC"),
    # grouped-query attention: the group letters trail Q's batch letters and do not index K, V
    ("rbgsd,bgtd,bgtd->rbgsd", "attention", "", "JA_ERR_SPEC"),
    ("bgsd,bgrtd,bgrtd->bgsd", "attention", "", "JA_ERR_SPEC"),
    ("bgrsd,bgsd,bgsd->bgrsd", "attention", "", "JA_ERR_SPEC"),
    # token-major relations: the letters before both position letters agree, and with the position and
    # head-dimension letters removed Q's letters are K's followed by the group letters
    ("bshd,bhtd,bhtd->bshd", "attention", "", "JA_ERR_SPEC"),
    ("bshd,bthd,bthd->bhsd", "attention", "", "JA_ERR_SPEC"),
    ("bsrgd,btgd,btgd->bsrgd", "attention", "", "JA_ERR_SPEC"),
    ("bshd,bthd,bthd->bshd", "attention", "causal=h,t", "JA_ERR_SPEC"),
    # fused contractions: the residual has the output's letters; the pair letter is B's last, nowhere else
    ("tm,mn->tn", "contract_add", "", "JA_ERR_SPEC"),
    ("tm,mn,nt->tn", "contract_add", "", "JA_ERR_SPEC"),
    ("td,dcf->tf", "contract_swiglu", "", "JA_ERR_SPEC"),
    ("tdc,dfc->tf", "contract_swiglu", "", "JA_ERR_SPEC"),
    ("td,dfc->tfc", "contract_swiglu", "", "JA_ERR_SPEC"),
    ("td,dfc,tf->tf", "contract_swiglu", "", "JA_ERR_SPEC"),
])
def test_spec_errors(B, einsum, op, params, code):
    with pytest.raises(B.JaError) as e:
        B.ja_spec_create(einsum, op, params)
    assert e.value.name == code
    assert B.ja_last_error()


@pytest.mark.parametrize("einsum", ["bshd,bthd,bthd->bshd", "bsgrd,btgd,btgd->bsgrd", "bhsd,bhtd,bhtd->bhsd",
                                    "bgrsd,bgtd,bgtd->bgrsd"])
def test_attention_spec_forms(B, orc, einsum):
    """Head-major and token-major attention specs (batch-head letters before
    or after the position letter) are accepted, and their causal tuple lists
    are the oracle's: the join does not depend on where the letters sit."""
    lq = einsum.split(",")[0]
    sp = {c: [0, 2] for c in einsum if c.isalpha()}
    sp.update({"s": [0, 128, 256, 300], "t": [0, 100, 300], "d": [0, 128], "r": [0, 1, 3]})
    letters, rec, seg = _tuples(B, einsum, "attention", sp, "causal=s,t")
    o_rec, o_seg = orc.tuple_records(list(letters), sp, group_by=list(lq), causal=("s", "t"))
    assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg)


def test_token_major_attention_has_no_unfused_path(B):
    """Blocks with batch-heads inside a row have the fused kernel only: the
    softmax aggregation writes rows in [batch-head][query] order."""
    from tensor_relational_join_amd.device import relation_for

    sp = {"b": [0, 1], "s": [0, 128, 256], "h": [0, 4], "t": [0, 128, 256], "d": [0, 128]}
    s = B.ja_spec_create("bshd,bthd,bthd->bshd", "attention", "causal=s,t")
    ls = B.ja_spec_letters(s)
    d = B.ja_decomp_create(s, [sp[c][-1] for c in ls], [len(sp[c]) - 1 for c in ls], [sp[c] for c in ls])
    try:
        ins = [relation_for(x, sp, B.JA_BF16) for x in ("bshd", "bthd", "bthd")]
        p = B.ja_plan_create(s, d, ins, relation_for("bshd", sp, B.JA_BF16))
        try:
            with pytest.raises(B.JaError) as e:
                B.ja_plan_partial_bytes(p)
            assert e.value.name == "JA_ERR_UNSUPPORTED"
        finally:
            B.ja_plan_destroy(p)
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)


def test_decomposition_errors(B):
    s = B.ja_spec_create("ij,jk->ik", "contract")
    try:
        for ext, iv, sp, code in [
            ([4, 4, 4], [5, 1, 1], None, "JA_ERR_DECOMP"),        # more intervals than cells
            ([4, 4, 4], [0, 1, 1], None, "JA_ERR_DECOMP"),
            ([4, 0, 4], [1, 1, 1], None, "JA_ERR_DECOMP"),
            ([4, 4, 4], [2, 1, 1], [[0, 3, 3], None, None], "JA_ERR_DECOMP"),   # not rising
            ([4, 4, 4], [2, 1, 1], [[0, 2, 5], None, None], "JA_ERR_DECOMP"),   # past the extent
        ]:
            with pytest.raises(B.JaError) as e:
                B.ja_decomp_create(s, ext, iv, sp)
            assert e.value.name == code
    finally:
        B.ja_spec_destroy(s)
    a = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t")
    try:
        with pytest.raises(B.JaError) as e:
            B.ja_decomp_create(a, [1, 1, 256, 128, 256], [1, 1, 2, 2, 2])  # letters b h s d t: d split
        assert e.value.name == "JA_ERR_DECOMP"
    finally:
        B.ja_spec_destroy(a)


def test_plan_validation_errors(B):
    from tensor_relational_join_amd.device import relation_for

    s = B.ja_spec_create("ij,jk->ik", "contract")
    sp = {"i": [0, 32, 64], "j": [0, 32, 64], "k": [0, 32, 64]}
    d = B.ja_decomp_create(s, [64, 64, 64], [2, 2, 2], [sp["i"], sp["j"], sp["k"]])
    try:
        A = relation_for("ij", sp, B.JA_F32)
        Bm = relation_for("jk", sp, B.JA_F32)
        C = relation_for("ik", sp, B.JA_F32)
        p = B.ja_plan_create(s, d, [A, Bm], C)
        assert B.ja_plan_device_bytes(p)[0] > 0
        with pytest.raises(B.JaError) as e:       # running before upload
            B.ja_plan_run(p, [16, 32], 48)
        assert e.value.name == "JA_ERR_STATE"
        B.ja_plan_destroy(p)
        # A blocked finer than the decomposition (a coarser blocking is read in sub-boxes)
        bad = B.Relation((64, 64), nblk=(4, 2), dtype=B.JA_F32)
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [bad, Bm], C)
        assert e.value.name == "JA_ERR_SHAPE"
        C16 = relation_for("ik", sp, B.JA_BF16)
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [A, Bm], C16)
        assert e.value.name == "JA_ERR_DTYPE"
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [A], C)
        assert e.value.name == "JA_ERR_ARG"
        A16, B16 = relation_for("ij", sp, B.JA_BF16), relation_for("jk", {**sp, "k": [0, 30, 64]}, B.JA_BF16)
        with pytest.raises(B.JaError):
            B.ja_plan_create(s, d, [A16, B16], C16)
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)


def test_contraction_operands_blocked_coarser(B):
    """A two-letter contraction operand may be blocked coarser than the
    decomposition (each of its split points one of the decomposition's): its
    tuples read sub-boxes of its blocks in place.  A blocking with a split
    point the decomposition lacks, or a batched operand blocked apart, is
    refused."""
    from tensor_relational_join_amd.device import relation_for

    sp = {"i": [0, 64, 128], "j": [0, 32, 64, 96, 128], "k": [0, 64, 128]}
    s = B.ja_spec_create("ij,jk->ik", "contract")
    d = B.ja_decomp_create(s, [128, 128, 128], [2, 4, 2], [sp["i"], sp["j"], sp["k"]])
    try:
        out = relation_for("ik", sp, B.JA_BF16)
        for aj, bj in (([0, 64, 128], [0, 128]), ([0, 128], [0, 32, 128]), (sp["j"], sp["j"])):
            a = relation_for("ij", {**sp, "j": aj}, B.JA_BF16)
            b = relation_for("jk", {**sp, "j": bj, "k": [0, 128]}, B.JA_BF16)
            B.ja_plan_destroy(B.ja_plan_create(s, d, [a, b], out))
        bad = relation_for("ij", {**sp, "j": [0, 48, 128]}, B.JA_BF16)
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [bad, relation_for("jk", sp, B.JA_BF16)], out)
        assert e.value.name == "JA_ERR_SHAPE"
        with pytest.raises(B.JaError) as e:  # the output stays blocked as the decomposition
            B.ja_plan_create(s, d, [relation_for("ij", sp, B.JA_BF16), relation_for("jk", sp, B.JA_BF16)],
                             relation_for("ik", {**sp, "k": [0, 128]}, B.JA_BF16))
        assert e.value.name == "JA_ERR_SHAPE"
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)
    bsp = {"b": [0, 1, 2], "i": [0, 64], "j": [0, 32, 64], "k": [0, 64]}
    s = B.ja_spec_create("bij,bjk->bik", "contract")
    d = B.ja_decomp_create(s, [2, 64, 64, 64], [2, 1, 2, 1], [bsp["b"], bsp["i"], bsp["j"], bsp["k"]])
    try:
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [relation_for("bij", {**bsp, "j": [0, 64]}, B.JA_BF16),
                                    relation_for("bjk", bsp, B.JA_BF16)], relation_for("bik", bsp, B.JA_BF16))
        assert e.value.name == "JA_ERR_SHAPE"
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)


def test_fused_contraction_plans(B):
    """contract_add and contract_swiglu: same tuples as the plain
    contraction; 16-bit relations only; the pair letter whole with extent 2;
    no unfused path; not planned by the logical optimizer."""
    from tensor_relational_join_amd.device import relation_for

    sp = {"t": [0, 64, 128], "m": [0, 64, 128], "n": [0, 32, 96]}
    plain = _tuples(B, "tm,mn->tn", "contract", sp)
    fused = _tuples(B, "tm,mn,tn->tn", "contract_add", sp)
    assert plain[0] == "tmn" and fused[0] == "tmn"
    assert np.array_equal(plain[1], fused[1]) and np.array_equal(plain[2], fused[2])
    s = B.ja_spec_create("tm,mn,tn->tn", "contract_add")
    d = B.ja_decomp_create(s, [128, 128, 96], [2, 2, 2], [sp["t"], sp["m"], sp["n"]])
    try:
        bf = [relation_for(x, sp, B.JA_BF16) for x in ("tm", "mn", "tn")]
        p = B.ja_plan_create(s, d, bf, relation_for("tn", sp, B.JA_BF16))
        for call in (lambda: B.ja_plan_partial_bytes(p), lambda: B.ja_kernel(p, [16, 32, 48], 64),
                     lambda: B.ja_agg(p, B.JA_AGG_SUM, 16, 32)):
            with pytest.raises(B.JaError) as e:
                call()
            assert e.value.name in ("JA_ERR_UNSUPPORTED", "JA_ERR_STATE")
        with pytest.raises(B.JaError) as e:
            B.ja_plan_partial_bytes(p)
        assert e.value.name == "JA_ERR_UNSUPPORTED"
        B.ja_plan_destroy(p)
        for ins, out, code in (
                (bf, relation_for("tn", sp, B.JA_F32), "JA_ERR_DTYPE"),                      # f32 output
                ([relation_for(x, sp, B.JA_F32) for x in ("tm", "mn", "tn")],
                 relation_for("tn", sp, B.JA_F32), "JA_ERR_DTYPE"),                           # f32 inputs
                (bf[:2] + [relation_for("tn", sp, B.JA_F16)], relation_for("tn", sp, B.JA_BF16), "JA_ERR_DTYPE"),
                (bf[:2] + [relation_for("tn", {**sp, "n": [0, 48, 96]}, B.JA_BF16)],
                 relation_for("tn", sp, B.JA_BF16), "JA_ERR_SHAPE")):                         # residual blocked apart
            with pytest.raises(B.JaError) as e:
                B.ja_plan_create(s, d, ins, out)
            assert e.value.name == code
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)
    sw = {"t": [0, 64, 128], "d": [0, 64], "f": [0, 48, 96], "c": [0, 2]}
    plain = _tuples(B, "td,df->tf", "contract", {k: sw[k] for k in "tdf"})
    fused = _tuples(B, "td,dfc->tf", "contract_swiglu", sw)
    assert fused[0] == "tdfc" and np.array_equal(plain[1], fused[1][:, :3]) and np.array_equal(plain[2], fused[2])
    s = B.ja_spec_create("td,dfc->tf", "contract_swiglu")
    try:
        d = B.ja_decomp_create(s, [128, 64, 96, 2], [2, 1, 2, 1], [sw["t"], sw["d"], sw["f"], sw["c"]])
        try:
            p = B.ja_plan_create(s, d, [relation_for("td", sw, B.JA_BF16), relation_for("dfc", sw, B.JA_BF16)],
                                 relation_for("tf", sw, B.JA_BF16))
            B.ja_plan_destroy(p)
        finally:
            B.ja_decomp_destroy(d)
        for ext, iv, splits in (([128, 64, 96, 4], [2, 1, 2, 1], [sw["t"], sw["d"], sw["f"], [0, 4]]),
                                ([128, 64, 96, 2], [2, 1, 2, 2], [sw["t"], sw["d"], sw["f"], [0, 1, 2]])):
            d = B.ja_decomp_create(s, ext, iv, splits)
            try:
                c = {"c": splits[3]}
                with pytest.raises(B.JaError) as e:
                    B.ja_plan_create(s, d, [relation_for("td", sw, B.JA_BF16),
                                            relation_for("dfc", {**sw, **c}, B.JA_BF16)],
                                     relation_for("tf", sw, B.JA_BF16))
                assert e.value.name == "JA_ERR_DECOMP"
            finally:
                B.ja_decomp_destroy(d)
        g = B.ja_graph_create()
        try:
            x = B.ja_graph_add_input(g, [128, 64])
            w = B.ja_graph_add_input(g, [64, 96, 2])
            with pytest.raises(B.JaError) as e:
                B.ja_graph_add_op(g, s, [x, w])
            assert e.value.name == "JA_ERR_UNSUPPORTED"
        finally:
            B.ja_graph_destroy(g)
    finally:
        B.ja_spec_destroy(s)


def test_bf16_alignment_is_refused_not_miscomputed(B):
    from tensor_relational_join_amd.device import relation_for

    s = B.ja_spec_create("ij,jk->ik", "contract")
    sp = {"i": [0, 16], "j": [0, 12], "k": [0, 16]}   # K = 12: not a multiple of 8
    d = B.ja_decomp_create(s, [16, 12, 16], [1, 1, 1], [sp["i"], sp["j"], sp["k"]])
    try:
        with pytest.raises(B.JaError) as e:
            B.ja_plan_create(s, d, [relation_for("ij", sp, B.JA_BF16), relation_for("jk", sp, B.JA_BF16)],
                             relation_for("ik", sp, B.JA_BF16))
        assert e.value.name == "JA_ERR_UNSUPPORTED"
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)


def test_operand_matrix_beyond_32bit_offsets_is_refused(B):
    """The MFMA contraction addresses every operand matrix with 32-bit buffer
    byte offsets: an operand block of 2^30 elements or more is refused at
    plan time (no kernel would address it), one just below is accepted."""
    from tensor_relational_join_amd.device import relation_for

    s = B.ja_spec_create("ij,jk->ik", "contract")
    try:
        for k, code in ((1 << 22, "JA_ERR_UNSUPPORTED"), ((1 << 22) - 8, None)):
            sp = {"i": [0, 256], "j": [0, k], "k": [0, 64]}
            d = B.ja_decomp_create(s, [256, k, 64], [1, 1, 1], [sp["i"], sp["j"], sp["k"]])
            try:
                ins = [relation_for("ij", sp, B.JA_BF16), relation_for("jk", sp, B.JA_BF16)]
                if code is None:
                    B.ja_plan_destroy(B.ja_plan_create(s, d, ins, relation_for("ik", sp, B.JA_BF16)))
                else:
                    with pytest.raises(B.JaError) as e:
                        B.ja_plan_create(s, d, ins, relation_for("ik", sp, B.JA_BF16))
                    assert e.value.name == code and "2^30" in str(e.value)
            finally:
                B.ja_decomp_destroy(d)
    finally:
        B.ja_spec_destroy(s)


def test_section_5_3_overlay_atom_count(B):
    g = json.load(open(os.path.join(GOLDEN, "section_5_3_overlay_atoms.json")))
    src = B.Relation(g["shape"], splits=[g["producer_row_splits"], g["col_splits"]], dtype=B.JA_BF16)
    dst = B.Relation(g["shape"], splits=[g["consumer_row_splits"], g["col_splits"]], dtype=B.JA_BF16)
    rp = B.ja_repart_create(src, dst)
    try:
        n_atoms, n_tasks = B.ja_repart_count(rp)
        assert n_atoms == g["n_atoms"]
        assert n_tasks >= n_atoms
    finally:
        B.ja_repart_destroy(rp)


def test_repartition_atoms_for_head_views(B):
    # token-major [8192, 12288] blocked 2x2 -> head-major [3,4,32,2048,128] blocks [1,1,1,128,128]
    src = B.Relation((8192, 12288), nblk=(2, 2), dtype=B.JA_BF16)
    dst = B.Relation((3, 4, 32, 2048, 128), nblk=(3, 4, 32, 16, 1), dtype=B.JA_BF16)
    view = B.make_view((4, 2048, 3, 32, 128), (2, 0, 3, 1, 4))
    rp = B.ja_repart_create(src, dst, view)
    try:
        assert B.ja_repart_count(rp) == (6144, 6144)
    finally:
        B.ja_repart_destroy(rp)
    # views that do not factor are refused
    bad = B.make_view((6, 4), (1, 0))
    with pytest.raises(B.JaError) as e:
        B.ja_repart_create(B.Relation((4, 6), nblk=(1, 1), dtype=B.JA_F32),
                           B.Relation((4, 6), nblk=(1, 1), dtype=B.JA_F32), bad)
    assert e.value.name == "JA_ERR_UNSUPPORTED"
    with pytest.raises(B.JaError) as e:
        B.ja_repart_create(B.Relation((4, 6), nblk=(1, 1), dtype=B.JA_F32),
                           B.Relation((4, 6), nblk=(1, 1), dtype=B.JA_BF16))
    assert e.value.name == "JA_ERR_DTYPE"


def test_repartition_views_with_unit_dimensions(B):
    # batch of one: the view's leading extent-1 axis indexes nothing
    src = B.Relation((256, 768), nblk=(2, 2), dtype=B.JA_BF16)
    dst = B.Relation((3, 1, 2, 256, 128), nblk=(3, 1, 2, 2, 1), dtype=B.JA_BF16)
    rp = B.ja_repart_create(src, dst, B.make_view((1, 256, 3, 2, 128), (2, 0, 3, 1, 4)))
    assert B.ja_repart_count(rp) == (12, 12)
    B.ja_repart_destroy(rp)
    rp = B.ja_repart_create(B.Relation((1, 1), nblk=(1, 1), dtype=B.JA_F32), B.Relation((1,), nblk=(1,), dtype=B.JA_F32),
                            B.make_view((1,), (0,)))
    assert B.ja_repart_count(rp) == (1, 1)
    B.ja_repart_destroy(rp)


def test_one_shot_entry_points_refuse_a_small_workspace(B):
    """ja_einsum and ja_repartition check the caller's workspace against the
    size query before any HIP call, so an undersized (or absent) workspace is
    refused on the host."""
    s = B.ja_spec_create("ij,jk->ik", "contract")
    d = B.ja_decomp_create(s, [64, 64, 64], [2, 2, 2])
    try:
        ins = [B.Relation((64, 64), nblk=(2, 2), dtype=B.JA_F32)] * 2
        out = B.Relation((64, 64), nblk=(2, 2), dtype=B.JA_F32)
        need = B.ja_einsum_workspace_bytes(s, d, ins, out)
        assert need > 0 and need % 256 == 0
        for ws, nbytes in ((0, need), (1 << 20, need - 1)):
            with pytest.raises(B.JaError) as e:
                B.ja_einsum(s, d, ins, [16, 16], out, 16, ws, nbytes)
            assert e.value.name == "JA_ERR_WORKSPACE"
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)
    src = B.Relation((256, 256), splits=[[0, 128, 256], [0, 256]], dtype=B.JA_BF16)
    dst = B.Relation((256, 256), splits=[[0, 64, 128, 192, 256], [0, 256]], dtype=B.JA_BF16)
    need = B.ja_repartition_workspace_bytes(src, dst)
    assert need > 0
    with pytest.raises(B.JaError) as e:
        B.ja_repartition(src, 16, dst, 16, None, 1 << 20, need - 1)
    assert e.value.name == "JA_ERR_WORKSPACE"


# ------------------------------------------------------------------ device-side join (host checks)

def test_device_join_sizes_and_errors(B):
    """ja_djoin_* host side: capacities from the interval counts, argument
    checks before anything reaches the GPU, decomposition rules."""
    s = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t")
    try:
        dj = B.ja_djoin_create(s, [2, 4, 2048, 128, 2048], [1, 4, 16, 1, 16])
        try:
            tb, wb, mt, ms, ns = B.ja_djoin_device_bytes(dj)
            assert (mt, ms, ns) == (4 * 16 * 16, 4 * 16, 2 + 5 + 17 + 2 + 17)
            assert tb >= 8 and wb >= 4 * (ms + 1)
            with pytest.raises(B.JaError) as e:  # table not uploaded
                B.ja_djoin_run(dj, 256, 256, 256, 256, 256)
            assert e.value.name == "JA_ERR_STATE"
        finally:
            B.ja_djoin_destroy(dj)
        ext = [2, 4, 2048, 128, 2048]
        for iv in ([1, 4, 16, 2, 16], [1, 5, 16, 1, 16], [0, 4, 16, 1, 16]):  # split d; 5 > 4 heads; no interval
            with pytest.raises(B.JaError) as e:
                B.ja_djoin_create(s, ext, iv)
            assert e.value.name == "JA_ERR_DECOMP"
        with pytest.raises(B.JaError) as e:  # 2^30 grid cells
            B.ja_djoin_create(s, [1 << 10, 1 << 10, 1 << 10, 128, 1 << 10], [1 << 10, 1 << 10, 1 << 5, 1, 1 << 5])
        assert e.value.name == "JA_ERR_UNSUPPORTED"
    finally:
        B.ja_spec_destroy(s)
    s = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "packed=1024,2560,4096")
    try:
        B.ja_djoin_destroy(B.ja_djoin_create(s, [1, 1, 4096, 128, 4096], [1, 1, 3, 1, 2]))
        for ext, iv in (([1, 1, 4096, 128, 4096], [1, 1, 4, 1, 2]),   # more intervals than sequences
                        ([1, 1, 4000, 128, 4000], [1, 1, 2, 1, 2])):  # does not span every sequence
            with pytest.raises(B.JaError) as e:
                B.ja_djoin_create(s, ext, iv)
            assert e.value.name == "JA_ERR_DECOMP"
    finally:
        B.ja_spec_destroy(s)


def test_packed_device_spec_and_planner_checks(B, orc):
    """"packed=device": the sequences end at the cuts of s (and t, cut
    alike).  The host join keeps the block-diagonal pairs; the device planner
    takes only such specs, head dimension 128, bf16 or fp16."""
    with pytest.raises(B.JaError) as e:
        B.ja_spec_create("ij,jk->ik", "contract", "packed=device")
    assert e.value.name == "JA_ERR_SPEC"
    cuts = [0, 300, 1000, 1024]
    splits = {"b": [0, 1], "h": [0, 2, 4], "s": cuts, "d": [0, 128], "t": cuts}
    letters, rec, seg = _tuples(B, "bhsd,bhtd,bhtd->bhsd", "attention", splits, "packed=device;causal=s,t")
    o_rec, o_seg = orc.tuple_records(list(letters), splits, group_by=list("bhsd"), causal=("s", "t"),
                                     packed=("s", "t", cuts[1:]))
    assert np.array_equal(rec, o_rec) and np.array_equal(seg, o_seg) and rec.shape[0] == 2 * 3
    s = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "packed=device;causal=s,t")
    try:
        with pytest.raises(B.JaError) as e:  # s and t cut differently
            B.ja_decomp_create(s, [1, 4, 1024, 128, 1024], [1, 1, 2, 1, 2],
                               [[0, 1], [0, 4], [0, 500, 1024], [0, 128], [0, 600, 1024]])
        assert e.value.name == "JA_ERR_DECOMP"
        da = B.ja_dattn_create(s, [1, 4, 1024, 128, 1024], [1, 2, 3, 1, 3])
        try:
            tb, wb, ns = B.ja_dattn_device_bytes(da)
            assert tb > 0 and wb > 0 and ns == 2 + 3 + 4 + 2 + 4
            with pytest.raises(B.JaError) as e:
                B.ja_dattn_run(da, 256, 256, 256, 256, 256, 256, 256)
            assert e.value.name == "JA_ERR_STATE"
        finally:
            B.ja_dattn_destroy(da)
        for ext, iv, dt, name in (([1, 4, 1024, 64, 1024], [1, 2, 3, 1, 3], B.JA_BF16, "JA_ERR_UNSUPPORTED"),
                                  ([1, 4, 1024, 128, 1024], [1, 2, 3, 1, 2], B.JA_BF16, "JA_ERR_DECOMP"),
                                  ([1, 4, 1024, 128, 1024], [1, 2, 3, 1, 3], B.JA_F32, "JA_ERR_DTYPE")):
            with pytest.raises(B.JaError) as e:
                B.ja_dattn_create(s, ext, iv, dt)
            assert e.value.name == name
    finally:
        B.ja_spec_destroy(s)
    s = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t")
    try:
        with pytest.raises(B.JaError) as e:
            B.ja_dattn_create(s, [1, 4, 1024, 128, 1024], [1, 2, 3, 1, 3])
        assert e.value.name == "JA_ERR_SPEC"
    finally:
        B.ja_spec_destroy(s)


def test_calibration_argument_checks(B):
    for wgs, iters, sink in ((0, 1, 256), (1, 0, 256), (1, 1, 0), (1, 1, 258)):
        with pytest.raises(B.JaError) as e:
            B.ja_calibrate_mfma(wgs, iters, sink)
        assert e.value.name == "JA_ERR_ARG"
    # the copy ceiling: NULL buffers, misaligned pointers or sizes are refused before any launch
    for src, dst, n in ((0, 256, 16), (256, 0, 16), (264, 256, 16), (256, 264, 16), (256, 512, 24)):
        with pytest.raises(B.JaError) as e:
            B.ja_calibrate_copy(src, dst, n)
        assert e.value.name == "JA_ERR_ARG"


def test_noalloc_einsum_refuses_a_plan_beyond_its_scratch(B):
    """ja_einsum_noalloc's tables live in a static device array of
    JA_NOALLOC_SCRATCH_BYTES: a plan that needs more is refused with
    JA_ERR_WORKSPACE before any HIP call (so this runs without a GPU).  A
    contraction cut into 100 x 100 x 100 blocks of 8 has 10^6 tuples of 40
    bytes of table each."""
    from tensor_relational_join_amd.device import relation_for

    s = B.ja_spec_create("ij,jk->ik", "contract")
    sp = {c: list(range(0, 801, 8)) for c in "ijk"}
    d = B.ja_decomp_create(s, [800] * 3, [100] * 3, [sp["i"], sp["j"], sp["k"]])
    try:
        ins = [relation_for("ij", sp, B.JA_BF16), relation_for("jk", sp, B.JA_BF16)]
        out = relation_for("ik", sp, B.JA_BF16)
        assert B.ja_einsum_workspace_bytes(s, d, ins, out) > B.JA_NOALLOC_SCRATCH_BYTES
        with pytest.raises(B.JaError) as e:
            B.ja_einsum_noalloc(s, d, ins, [256, 256], out, 256)
        assert e.value.name == "JA_ERR_WORKSPACE" and "static scratch" in str(e.value)
    finally:
        B.ja_decomp_destroy(d)
        B.ja_spec_destroy(s)
