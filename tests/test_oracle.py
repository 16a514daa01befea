"""Pins of the CPU oracle against facts fixed by the pages and by mathematics:
the pages' worked examples (golden fixtures), closed forms, brute force on
tiny inputs, an independent library routine, and invariants.  Each test is
chosen so that a plausible mistake in the oracle (dropped term, wrong index,
transposed operand, off-by-one mask, wrong rounding) fails at least one."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from tensor_relational_join_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints(rng, shape, lo=-3, hi=4):
    # small integers: every sum of products is exact in float64, in any order
    return rng.integers(lo, hi, size=shape).astype(np.float64)


# ---------------------------------------------------------------- bfloat16

def test_bf16_known_encodings(orc):
    cases = {
        1.0: 0x3F80, -1.0: 0xBF80, 0.0: 0x0000, 2.0: 0x4000, 0.5: 0x3F00,
        1.0 + 2.0 ** -8: 0x3F80,          # halfway between 1 and 1+2^-7: ties to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # halfway between 1+2^-7 and 1+2^-6: ties to even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above halfway: rounds up
        2.0 ** -133: 0x0001,              # smallest subnormal
        2.0 ** -134: 0x0000,              # half the smallest subnormal: ties to even (zero)
        3 * 2.0 ** -134: 0x0002,          # 1.5 * smallest subnormal: ties to even (2)
        2.0 ** -126: 0x0080,              # smallest normal
        3.3895313892515355e38: 0x7F7F,    # largest finite bf16
        3.4e38: 0x7F80,                   # beyond the largest finite value's rounding range
        float("inf"): 0x7F80, float("-inf"): 0xFF80,
    }
    xs = np.array(list(cases.keys()))
    got = orc.f64_to_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == cases[float(x)], (x, hex(int(g)))
    assert orc.f64_to_bf16(np.array([np.nan]))[0] & 0x7FFF > 0x7F80


def test_bf16_all_patterns_roundtrip(orc):
    h = np.arange(65536, dtype=np.uint16)
    v = orc.bf16_to_f64(h)
    finite = ~np.isnan(v)
    back = orc.f64_to_bf16(v)
    ok = (back == h) | ~finite
    # -0.0 must keep its sign bit
    assert np.all(ok)
    # decode agrees with widening the bits into a float32 (independent route)
    with np.errstate(invalid="ignore"):
        w = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(v[finite], w[finite])


def test_bf16_rounding_vs_independent_float32_route(orc):
    # for values exactly representable in float32, rounding from float64 must
    # equal the bit-trick rounding of the float32 (a second implementation)
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    f = f[np.abs(f) < 3.0e38]
    a = orc.f64_to_bf16(f.astype(np.float64))
    b = synth.f32_to_bf16_bits(f)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- einsum

SPECS = [
    ("ij,jk->ik", {"i": 3, "j": 4, "k": 5}),
    ("ij,kj->ik", {"i": 3, "j": 4, "k": 2}),      # second operand transposed
    ("ji,jk->ik", {"i": 2, "j": 5, "k": 3}),      # first operand transposed
    ("bij,bjk->bik", {"b": 2, "i": 3, "j": 2, "k": 3}),
    ("bhsd,bhtd->bhst", {"b": 1, "h": 2, "s": 3, "t": 4, "d": 2}),
    ("bhst,bhtd->bhsd", {"b": 2, "h": 1, "s": 2, "t": 3, "d": 2}),
    ("i,j->ij", {"i": 3, "j": 4}),                # outer product, nothing summed
    ("ij,j->i", {"i": 4, "j": 3}),
]


def _operands(spec, ext, rng):
    ins, _ = spec.split("->")[0].split(","), None
    return [_ints(rng, tuple(ext[c] for c in s)) for s in ins]


@pytest.mark.parametrize("spec,ext", SPECS)
def test_einsum_equals_brute_force_relational(orc, spec, ext):
    rng = np.random.default_rng(len(spec))
    A, B = _operands(spec, ext, rng)
    assert np.array_equal(orc.einsum(spec, A, B), orc.brute_force_einsum(spec, A, B))


@pytest.mark.parametrize("spec,ext", SPECS)
def test_einsum_vs_numpy_library(orc, spec, ext):
    rng = np.random.default_rng(7)
    A, B = [rng.standard_normal(x.shape) for x in _operands(spec, ext, rng)]
    np.testing.assert_allclose(orc.einsum(spec, A, B), np.einsum(spec, A, B), rtol=1e-13, atol=1e-13)


def test_einsum_closed_forms(orc):
    M, K, N = 5, 7, 3
    ones = orc.einsum("ij,jk->ik", np.ones((M, K)), np.ones((K, N)))
    assert np.all(ones == K)
    B = np.arange(K * N, dtype=np.float64).reshape(K, N)
    assert np.array_equal(orc.einsum("ij,jk->ik", np.eye(K), B), B)
    # a one-hot row of A picks one row of B: catches a transposed operand
    A = np.zeros((2, K)); A[0, 4] = 1; A[1, 2] = 2
    C = orc.einsum("ij,jk->ik", A, B)
    assert np.array_equal(C[0], B[4]) and np.array_equal(C[1], 2 * B[2])


def test_einsum_points_match_full(orc):
    rng = np.random.default_rng(3)
    A, B = rng.standard_normal((6, 9)), rng.standard_normal((9, 5))
    full = orc.einsum("ij,jk->ik", A, B)
    pts = np.array([[0, 0], [5, 4], [2, 3], [3, 0]])
    assert np.array_equal(orc.einsum_points("ij,jk->ik", A, B, pts), full[tuple(pts.T)])


def test_matmul_matches_brute_force(orc):
    rng = np.random.default_rng(4)
    A, B = _ints(rng, (4, 6)), _ints(rng, (6, 3))
    assert np.array_equal(orc.matmul(A, B), orc.brute_force_einsum("ij,jk->ik", A, B))


# ---------------------------------------------------------------- join-agg specs

def test_examples_3_8_and_3_9_specs(orc):
    g = json.load(open(os.path.join(GOLDEN, "example_3_8_3_9_matmul_specs.json")))
    for case in g["cases"]:
        specs = orc.joinagg_spec("ij,jk->ik", case["splits"])
        assert len(specs) == case["n_specs"]
        got = [{"A": [list(F.inputs[0][0]), list(F.inputs[0][1])],
                "B": [list(F.inputs[1][0]), list(F.inputs[1][1])],
                "C": [list(F.output[0]), list(F.output[1])]} for F in specs]
        assert got == case["specs"]
        outs = []
        for F in specs:
            if [list(F.output[0]), list(F.output[1])] not in outs:
                outs.append([list(F.output[0]), list(F.output[1])])
        assert outs == case["distinct_outputs"]
        assert orc.tiles([tuple(map(tuple, o)) for o in outs], [256, 256])
        letters = ["i", "j", "k"]
        _, seg = orc.tuple_records(letters, case["splits"], group_by=["i", "k"])
        assert list(np.diff(seg)) == case["segment_sizes"]


def test_spec_count_is_product_of_intervals(orc):
    rng = np.random.default_rng(11)
    ext = {"i": 12, "j": 10, "k": 9}
    for _ in range(20):
        q = {c: int(rng.integers(1, 5)) for c in ext}
        splits = {c: orc.equal_splits(ext[c], q[c]) for c in ext}
        specs = orc.joinagg_spec("ij,jk->ik", splits)
        assert len(specs) == q["i"] * q["j"] * q["k"]
        # distinct output types form a tiling of the output (tiling condition)
        outs = list({F.output for F in specs})
        assert len(outs) == q["i"] * q["k"]
        assert orc.tiles(outs, [12, 9])


def test_equal_splits_reading(orc):
    assert orc.equal_splits(10, 3) == [0, 4, 7, 10]
    assert orc.equal_splits(2752 * 4, 4) == [0, 2752, 5504, 8256, 11008]
    assert orc.equal_splits(7, 7) == list(range(8))


def test_tiling_condition_detects_overlap_and_gap(orc):
    assert orc.tiles([((0, 0), (2, 4)), ((2, 0), (4, 4))], [4, 4])
    assert not orc.tiles([((0, 0), (3, 4)), ((2, 0), (4, 4))], [4, 4])   # overlap
    assert not orc.tiles([((0, 0), (2, 4)), ((3, 0), (4, 4))], [4, 4])   # gap
    # a join-agg whose output types overlap must be refused at recompose
    specs = [orc.FunctionSpec({}, [((0,), (2,))], ((0,), (2,))),
             orc.FunctionSpec({}, [((1,), (3,))], ((1,), (3,)))]
    with pytest.raises(ValueError):
        orc.execute_joinagg(specs, [np.arange(3.0)], [3], lambda a: a, np.add)


@pytest.mark.parametrize("spec,ext", SPECS[:6])
def test_decomposition_invariance_exact(orc, spec, ext):
    """Every decomposition of the same einsum gives the same result; with
    small-integer inputs the sums are exact, so equality is bitwise."""
    rng = np.random.default_rng(5)
    A, B = _operands(spec, ext, rng)
    dense = orc.einsum(spec, A, B)
    for _ in range(6):
        splits = {}
        for c, n in ext.items():
            k = int(rng.integers(0, n))
            pts = sorted(set([0, n] + list(rng.choice(np.arange(1, n), size=min(k, n - 1), replace=False)))) \
                if n > 1 else [0, n]
            splits[c] = [int(p) for p in pts]
        assert np.array_equal(orc.contract_joinagg(spec, A, B, splits), dense)


def test_config_tuple_counts(orc):
    # 2x2x2 matmul: 8 tuples, 4 segments of 2
    sp = {c: orc.equal_splits(64, 2) for c in "ijk"}
    rec, seg = orc.tuple_records(list("ijk"), sp, group_by=["i", "k"])
    assert rec.shape[0] == 8 and len(seg) - 1 == 4 and set(np.diff(seg)) == {2}
    # FFN contraction: b by 2, d by 4, f by 4 -> 32 tuples, 8 segments of 4
    sp = {"b": orc.equal_splits(2048, 2), "d": orc.equal_splits(4096, 4), "f": orc.equal_splits(11008, 4)}
    rec, seg = orc.tuple_records(list("bdf"), sp, group_by=["b", "f"])
    assert rec.shape[0] == 32 and len(seg) - 1 == 8 and set(np.diff(seg)) == {4}
    # causal attention, 16 blocks of 128 on s and t: n(n+1)/2 = 136 tuples per (b, h)
    sp = {"b": [0, 1, 2, 3, 4], "h": list(range(33)), "s": orc.equal_splits(2048, 16),
          "t": orc.equal_splits(2048, 16), "d": [0, 128]}
    rec, seg = orc.tuple_records(list("bhsdt"), sp, group_by=list("bhsd"), causal=("s", "t"))
    assert rec.shape[0] == 4 * 32 * 136 == 17408
    assert len(seg) - 1 == 2048
    lens = np.diff(seg).reshape(4, 32, 16)
    assert np.all(lens == np.arange(1, 17)[None, None, :])


def test_causal_drop_is_exact(orc):
    """A tuple is kept iff at least one (s, t) pair in its cell has t <= s
    (checked cell by cell on uneven intervals)."""
    s_sp, t_sp = [0, 3, 4, 9, 12], [0, 2, 5, 6, 12]
    rec, _ = orc.tuple_records(["s", "t"], {"s": s_sp, "t": t_sp}, group_by=["s"], causal=("s", "t"))
    kept = {tuple(r) for r in rec.tolist()}
    for si, ti in itertools.product(range(4), range(4)):
        visible = any(t <= s for s in range(s_sp[si], s_sp[si + 1]) for t in range(t_sp[ti], t_sp[ti + 1]))
        assert ((si, ti) in kept) == visible


def test_tuple_record_order(orc):
    rec, seg = orc.tuple_records(list("ijk"), {"i": [0, 1, 2], "j": [0, 1, 2, 3], "k": [0, 1, 2]},
                                 group_by=["i", "k"])
    # sorted by (i, k), then j
    keys = [(r[0], r[2], r[1]) for r in rec.tolist()]
    assert keys == sorted(keys)
    assert list(seg) == [0, 3, 6, 9, 12]


# ---------------------------------------------------------------- attention

def test_attention_hand_example(orc):
    # one query, two keys: scores (1, 0) -> weights (e, 1)/(e + 1)
    Q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    K = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 1, 2, 2)
    V = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 1, 2, 2)
    e = math.e
    want = np.array([(e + 3) / (e + 1), (2 * e + 4) / (e + 1)])
    got = orc.attention(Q, K, V, 1.0, False).reshape(2)
    np.testing.assert_allclose(got, want, rtol=1e-15)
    # the scale multiplies the scores before the softmax: scores (2, 0) * 0.5
    got = orc.attention(2 * Q, K, V, 0.5, False).reshape(2)
    np.testing.assert_allclose(got, want, rtol=1e-15)


def test_attention_causal_prefix_mean(orc):
    # zero queries give equal scores: row s averages V over keys 0..s inclusive
    rng = np.random.default_rng(2)
    S, D = 7, 3
    V = rng.standard_normal((1, 2, S, D))
    K = rng.standard_normal((1, 2, S, D))
    Q = np.zeros((1, 2, S, D))
    out = orc.attention(Q, K, V, 0.3, True)
    want = np.cumsum(V, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)
    out = orc.attention(Q, K, V, 0.3, False)
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=2, keepdims=True), out.shape), rtol=1e-14)


def test_attention_first_row_is_first_value(orc):
    rng = np.random.default_rng(9)
    Q, K, V = (rng.standard_normal((2, 3, 5, 4)) for _ in range(3))
    out = orc.attention(Q, K, V, 0.5, True)
    np.testing.assert_allclose(out[:, :, 0], V[:, :, 0], rtol=1e-15)


def test_attention_dominant_key(orc):
    # a key aligned with the query and a huge scale puts all weight on it
    Q = np.zeros((1, 1, 3, 2)); Q[0, 0, 2] = [1.0, 0.0]
    K = np.array([[0.0, 1.0], [1.0, 0.0], [0.0, -1.0]]).reshape(1, 1, 3, 2)
    V = np.array([[10.0, 0.0], [0.0, 20.0], [5.0, 5.0]]).reshape(1, 1, 3, 2)
    out = orc.attention(Q, K, V, 1000.0, True)
    np.testing.assert_allclose(out[0, 0, 2], [0.0, 20.0], atol=1e-12)


def test_gqa_hand_example(orc):
    """Grouped-query attention (the pages' section 3.3): two query heads share
    one key-value head.  One query per head, two keys, scale 1: head 0's
    query (1, 0) scores the keys (1, 0); head 1's query (0, 1) scores them
    (0, 1).  Both read the same V."""
    Q = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    K = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 1, 2, 2)
    V = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 1, 2, 2)
    e = math.e
    want = np.array([[(e + 3) / (e + 1), (2 * e + 4) / (e + 1)],
                     [(1 + 3 * e) / (1 + e), (2 + 4 * e) / (1 + e)]])
    got = orc.attention(Q, K, V, 1.0, False).reshape(2, 2)
    np.testing.assert_allclose(got, want, rtol=1e-15)


def test_gqa_equals_mha_on_repeated_kv(orc):
    """Query heads g*4 .. g*4+3 use key-value head g: the same as multi-head
    attention with every key-value head repeated four times (a wrong head
    map, such as h mod HK, fails this)."""
    rng = np.random.default_rng(31)
    B, HK, R, S, D = 2, 3, 4, 17, 8
    Q = rng.standard_normal((B, HK * R, S, D))
    K, V = (rng.standard_normal((B, HK, S, D)) for _ in range(2))
    Kr, Vr = np.repeat(K, R, axis=1), np.repeat(V, R, axis=1)
    for causal in (True, False):
        got = orc.attention(Q, K, V, 0.4, causal)
        want = orc.attention(Q, Kr, Vr, 0.4, causal)
        np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)
        blocked = orc.attention_online_blocked(Q, K, V, [0, 5, 17], [0, 8, 11, 17], 0.4, causal)
        np.testing.assert_allclose(blocked, want, rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        orc.attention(Q[:, :10], K, V, 0.4, True)  # 3 key-value heads do not divide 10 query heads


def test_gqa_tuple_count(orc):
    """Q [b, g, r, s, d] against K, V [b, g, t, d]: one tuple per (b, g, r,
    s, t) interval cell with t_lo < s_hi, so 16 query and key blocks give
    n (n + 1) / 2 = 136 tuples per (b, g, r) block and one segment per
    (b, g, r, s) block."""
    sp = {"b": [0, 1], "g": orc.equal_splits(8, 8), "r": [0, 4], "s": orc.equal_splits(2048, 16),
          "t": orc.equal_splits(2048, 16), "d": [0, 128]}
    rec, seg = orc.tuple_records("bgrsdt", sp, "bgrs", causal=("s", "t"))
    assert rec.shape == (8 * 136, 6) and len(seg) - 1 == 8 * 16


def test_attention_online_blocked_equals_two_pass(orc):
    rng = np.random.default_rng(12)
    S, D = 20, 4
    Q, K, V = (rng.standard_normal((1, 2, S, D)) for _ in range(3))
    ref = orc.attention(Q, K, V, 0.7, True)
    s_sp, t_sp = [0, 6, 13, 20], [0, 4, 9, 16, 20]
    for order in (None, lambda ts: ts[::-1], lambda ts: ts[1::2] + ts[0::2]):
        got = orc.attention_online_blocked(Q, K, V, s_sp, t_sp, 0.7, True, t_order=order)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # one tuple covering everything: the online form degenerates to plain softmax
    got = orc.attention_online_blocked(Q, K, V, [0, S], [0, S], 0.7, True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_attention_triples_pins(orc):
    """Per-tuple triples (the join's output before aggregation) pinned three
    ways: (1) each tuple's log-sum-exp m + ln l and normalised values acc / l
    equal scipy's logsumexp and a softmax over that tuple's visible scores
    (library routines, not this code); (2) their fold with the softmax
    aggregation, in any order, gives textbook two-pass attention; (3) the
    tuple list is the one the join keeps (causal drop, packed sequences)."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(21)
    S, D = 20, 4
    Q = rng.standard_normal((1, 4, S, D))
    K, V = (rng.standard_normal((1, 2, S, D)) for _ in range(2))  # two query heads per key-value head
    s_sp, t_sp = [0, 6, 13, 20], [0, 4, 9, 16, 20]
    for causal, ends in ((True, None), (False, None), (True, [7, 15, 20]), (False, [7, 15, 20])):
        tri = orc.attention_triples(Q, K, V, s_sp, t_sp, 0.7, causal, ends)
        keys = [k for k, *_ in tri]
        recs, _ = orc.tuple_records("bhst", {"b": [0, 1], "h": [0, 1, 2, 3, 4], "s": s_sp, "t": t_sp}, "bhs",
                                    causal=("s", "t") if causal else None,
                                    packed=("s", "t", ends) if ends else None)
        assert keys == [tuple(int(x) for x in r) for r in recs]
        seq = np.searchsorted(ends, np.arange(S), side="right") if ends else np.zeros(S, dtype=int)
        for (b, h, si, ti), m, l, acc in tri:
            for r, s_ in enumerate(range(s_sp[si], s_sp[si + 1])):
                ks = [t for t in range(t_sp[ti], t_sp[ti + 1]) if (not causal or t <= s_) and seq[t] == seq[s_]]
                if not ks:
                    assert m[r] == -np.inf and l[r] == 0 and not acc[r].any()
                    continue
                sc = 0.7 * K[b, h // 2, ks] @ Q[b, h, s_]
                assert abs(m[r] + np.log(l[r]) - logsumexp(sc)) < 1e-12
                np.testing.assert_allclose(acc[r] / l[r], softmax(sc) @ V[b, h // 2, ks], rtol=1e-12, atol=1e-13)
        ref = orc.attention(Q, K, V, 0.7, causal, ends)
        for order in (lambda x: x, lambda x: x[::-1], lambda x: x[1::2] + x[0::2]):
            out = np.zeros_like(Q)
            for b, h, si in {k[:3] for k in keys}:
                group = order([(m, l, a) for k, m, l, a in tri if k[:3] == (b, h, si)])
                m, l, acc = orc.softmax_fold(group)
                out[b, h, s_sp[si]:s_sp[si + 1]] = acc / l[:, None]
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_softmax_fold_identity_and_shift(orc):
    """The identity (-inf, 0, 0) leaves a triple unchanged, and a triple is
    the same element of the monoid under a change of reference maximum:
    (m, l, acc) ~ (m', l e^(m - m'), acc e^(m - m'))."""
    m, l, acc = np.array([0.5, -np.inf]), np.array([2.0, 0.0]), np.array([[1.0, -2.0], [0.0, 0.0]])
    ident = (np.full(2, -np.inf), np.zeros(2), np.zeros((2, 2)))
    for seq in ([(m, l, acc), ident], [ident, (m, l, acc)]):
        fm, fl, fa = orc.softmax_fold(seq)
        np.testing.assert_array_equal(fm, m)
        np.testing.assert_array_equal(fl, l)
        np.testing.assert_array_equal(fa, acc)
    other = (np.array([1.0, 3.0]), np.array([1.5, 4.0]), np.array([[0.25, 0.5], [1.0, 2.0]]))
    fm, fl, fa = orc.softmax_fold([(m, l, acc), other])
    fm2, fl2, fa2 = orc.softmax_fold([(m - 3.0, l * np.exp(3.0), acc * np.exp(3.0)), other])
    np.testing.assert_allclose(fa / fl[:, None], fa2 / fl2[:, None], rtol=1e-14)
    np.testing.assert_allclose(fm + np.log(fl), fm2 + np.log(fl2), rtol=1e-14)


# ---------------------------------------------------------------- rmsnorm / swiglu / add

def test_rmsnorm_hand_values(orc):
    y = orc.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 8 / r]], rtol=1e-15)
    # eps sits inside the square root
    y = orc.rmsnorm(np.array([[1.0, 1.0]]), np.array([1.0, 1.0]), 3.0)
    np.testing.assert_allclose(y, [[0.5, 0.5]], rtol=1e-15)
    # constant rows normalise to the gain times the sign
    g = np.array([0.5, 1.5, -2.0, 1.0])
    y = orc.rmsnorm(np.array([[7.0] * 4, [-0.25] * 4]), g, 0.0)
    np.testing.assert_allclose(y, [g, -g], rtol=1e-15)
    # the mean runs over the whole row (not per block): doubling D with zeros halves the mean
    y = orc.rmsnorm(np.array([[2.0, 0.0]]), np.array([1.0, 1.0]), 0.0)
    np.testing.assert_allclose(y, [[math.sqrt(2.0), 0.0]], rtol=1e-15)


def test_swiglu_hand_values(orc):
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    u = np.array([3.0, 2.0, 2.0, 0.5, 1.0])
    want = [0.0, 2.0 / (1.0 + math.exp(-1.0)), -2.0 / (1.0 + math.e), 20.0, -40.0 / (1.0 + math.exp(40.0))]
    np.testing.assert_allclose(orc.swiglu(g, u), want, rtol=1e-15)
    assert np.array_equal(orc.add(np.array([1.5, -2.0]), np.array([0.25, 2.0])), [1.75, 0.0])


# ---------------------------------------------------------------- relations and repartition

def test_relation_pack_unpack_and_order(orc):
    x = np.arange(6 * 5).reshape(6, 5)
    rel = orc.Relation(x.shape, [[0, 2, 6], [0, 3, 5]])
    flat = rel.pack(x)
    # block (0,0) rows 0-1 cols 0-2, then (0,1) rows 0-1 cols 3-4, then (1,0) ...
    assert list(flat[:6]) == [0, 1, 2, 5, 6, 7]
    assert list(flat[6:10]) == [3, 4, 8, 9]
    assert list(flat[10:13]) == [10, 11, 12]
    assert np.array_equal(rel.unpack(flat), x)


def test_repartition_elementwise_definition(orc):
    """Check the vectorised repartition against per-element index arithmetic."""
    rng = np.random.default_rng(6)
    src = orc.Relation((4, 6), [[0, 1, 4], [0, 4, 6]])
    dst = orc.Relation((2, 3, 4), [[0, 2], [0, 1, 3], [0, 3, 4]])
    x = rng.integers(0, 1000, size=(4, 6))
    vshape, perm = (4, 2, 3), (1, 2, 0)     # [4,2,3] -> [2,3,4]
    got = orc.repartition(src, src.pack(x), dst, vshape, perm)
    # per destination element: dst logical (a,b,c) = view (c,a,b) = src linear c*6 + a*3 + b
    want_dense = np.empty((2, 3, 4), dtype=x.dtype)
    for a, b, c in itertools.product(range(2), range(3), range(4)):
        lin = c * 6 + a * 3 + b
        want_dense[a, b, c] = x[lin // 6, lin % 6]
    assert np.array_equal(dst.unpack(got), want_dense)
    # round trip through another blocking is the identity
    mid = orc.Relation((4, 6), [[0, 3, 4], [0, 1, 2, 6]])
    back = orc.repartition(mid, orc.repartition(src, src.pack(x), mid), src)
    assert np.array_equal(back, src.pack(x))


def test_section_5_3_overlay(orc):
    g = json.load(open(os.path.join(GOLDEN, "section_5_3_overlay_atoms.json")))
    atoms = orc.overlay_atoms([g["producer_row_splits"], g["col_splits"]],
                              [g["consumer_row_splits"], g["col_splits"]])
    assert atoms[0] == g["atom_row_splits"]
    assert (len(atoms[0]) - 1) * (len(atoms[1]) - 1) == g["n_atoms"]
    # each producer block is the union of the listed atoms
    for pb, members in enumerate(g["producer_block_atoms"]):
        lo, hi = g["producer_row_splits"][pb], g["producer_row_splits"][pb + 1]
        inside = [a for a in range(len(atoms[0]) - 1) if atoms[0][a] >= lo and atoms[0][a + 1] <= hi]
        assert inside == members


# ---------------------------------------------------------------- the block

def _tiny_block(seed, T=12, Dm=8, heads=2, F=6, batch=2):
    rng = np.random.default_rng(seed)
    r = lambda a: rng.standard_normal(a) * 0.5
    return dict(x=r((T, Dm)), g1=1 + 0.1 * r(Dm), w_qkv=r((Dm, 3 * Dm)), w_o=r((Dm, Dm)), g2=1 + 0.1 * r(Dm),
                w_gate=r((Dm, F)), w_up=r((Dm, F)), w_down=r((F, Dm))), batch, T // batch, heads


def test_block_zero_weights_is_identity(orc):
    w, batch, seq, heads = _tiny_block(1)
    x = orc.round_bf16(w["x"])
    w = {k: (np.zeros_like(v) if k in ("w_o", "w_down") else v) for k, v in w.items()}
    w["x"] = x
    y = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    assert np.array_equal(y, x)


def test_block_causal_and_batch_independent(orc):
    w, batch, seq, heads = _tiny_block(2)
    y0 = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    w2 = dict(w); x = w["x"].copy()
    x[seq - 1] += 3.0          # last token of batch 0
    w2["x"] = x
    y1 = orc.llama_block(**w2, batch=batch, seq=seq, heads=heads)
    assert np.array_equal(y0[: seq - 1], y1[: seq - 1])      # earlier tokens unaffected
    assert np.array_equal(y0[seq:], y1[seq:])                # other batch unaffected
    assert not np.array_equal(y0[seq - 1], y1[seq - 1])


def test_block_heads_are_column_groups(orc):
    """Head h reads columns [h*hd, (h+1)*hd) of each third of W_qkv: zeroing
    head 1's value columns zeroes exactly head 1's output columns of the
    attention result (its slice of the W_o input)."""
    w, batch, seq, heads = _tiny_block(3)
    Dm = w["x"].shape[1]
    hd = Dm // heads
    w["w_qkv"][:, 2 * Dm + hd: 2 * Dm + 2 * hd] = 0.0
    _, mid = orc.llama_block(**w, batch=batch, seq=seq, heads=heads, return_intermediates=True)
    O = mid["O"]                    # [b, h, s, hd]
    assert np.all(O[:, 1] == 0.0) and np.any(O[:, 0] != 0.0)


def test_block_tokens_match_full(orc):
    w, batch, seq, heads = _tiny_block(4)
    y = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    toks = [0, 3, seq - 1, seq, seq + 2]
    yt = orc.llama_block_tokens(**w, batch=batch, seq=seq, heads=heads, tokens=toks)
    assert np.array_equal(yt, y[toks])


def test_contract_residual_rounds_once(orc):
    """A B + R with nothing rounded in between.  Small integers: the exact
    brute-force value.  The tie case: A B = 2^-8 + 2^-16 needs nine
    significant bits; rounded first to bf16 it becomes 2^-8 (a tie, to even)
    and 1 + 2^-8 is again a tie that goes to 1, while the unrounded sum
    1 + 2^-8 + 2^-16 rounds up to 1 + 2^-7."""
    rng = np.random.default_rng(11)
    A = rng.integers(-3, 4, (5, 7)).astype(np.float64)
    Bm = rng.integers(-3, 4, (7, 6)).astype(np.float64)
    R = rng.integers(-9, 10, (5, 6)).astype(np.float64)
    assert np.array_equal(orc.contract_residual("ij,jk->ik", A, Bm, R),
                          orc.brute_force_einsum("ij,jk->ik", A, Bm) + R)
    A = np.array([[1.0, 1.0]])
    Bm = np.array([[2.0 ** -8], [2.0 ** -16]])
    R = np.array([[1.0]])
    once = orc.round_bf16(orc.contract_residual("ij,jk->ik", A, Bm, R))
    twice = orc.round_bf16(orc.add(orc.round_bf16(orc.einsum("ij,jk->ik", A, Bm)), R))
    assert once[0, 0] == 1.0 + 2.0 ** -7 and twice[0, 0] == 1.0


def test_contract_swiglu_pair_order(orc):
    """Member 0 of the pair is the gate, member 1 the up projection.  With
    the up weights reading a column of ones, the result is silu of the gate:
    silu(ln 3) = ln 3 / (1 + 1/3) = 0.75 ln 3, silu(0) = 0; swapping the
    members would give silu(1) * ln 3 instead."""
    l3 = np.log(3.0)
    A = np.array([[l3, 1.0], [0.0, 1.0]])            # rows: (x, 1)
    W = np.zeros((2, 1, 2))
    W[0, 0, 0] = 1.0                                 # gate = x
    W[1, 0, 1] = 1.0                                 # up = 1
    h = orc.contract_swiglu("td,dfc->tf", A, W)
    assert abs(h[0, 0] - 0.75 * l3) < 1e-15 and h[1, 0] == 0.0
    # a wider case equals silu(A Wg) * (A Wu) from the separate contractions
    rng = np.random.default_rng(12)
    A = rng.standard_normal((4, 6))
    Wg, Wu = rng.standard_normal((6, 5)), rng.standard_normal((6, 5))
    h = orc.contract_swiglu("td,dfc->tf", A, np.stack([Wg, Wu], axis=2))
    assert np.array_equal(h, orc.swiglu(orc.matmul(A, Wg), orc.matmul(A, Wu)))


def test_fused_block_rounding_points(orc):
    """The fused block (adds and SwiGLU applied inside the contractions)
    rounds fewer intermediates: with zero projections it is still the
    identity, token rows still agree with the full block bit for bit, its
    intermediates a, gate, up and d are the unrounded contraction results,
    and it differs from the unfused block by no more than bf16 rounding."""
    w, batch, seq, heads = _tiny_block(5)
    w["x"] = orc.round_bf16(w["x"])
    z = {k: (np.zeros_like(v) if k in ("w_o", "w_down") else v) for k, v in w.items()}
    assert np.array_equal(orc.llama_block(**z, batch=batch, seq=seq, heads=heads, fused=True), w["x"])
    y, mid = orc.llama_block(**w, batch=batch, seq=seq, heads=heads, fused=True, return_intermediates=True)
    toks = [0, 2, seq - 1, seq + 1]
    yt = orc.llama_block_tokens(**w, batch=batch, seq=seq, heads=heads, tokens=toks, fused=True)
    assert np.array_equal(yt, y[toks])
    for k in ("a", "gate", "up", "d"):
        assert not np.array_equal(mid[k], orc.round_bf16(mid[k]))
    for k in ("h1", "qkv", "O", "x2", "h2", "f"):
        assert np.array_equal(mid[k], orc.round_bf16(mid[k]))
    yu = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    assert not np.array_equal(y, yu)
    assert np.linalg.norm(y - yu) <= 2.0 ** -7 * np.linalg.norm(yu)


def test_block_in_ieee_half(orc):
    """The block with every materialised relation rounded to IEEE half
    instead of bf16.  Half keeps 11 significant bits to bf16's 8: against
    the same chain with no rounding at all, the half block sits roughly 8
    times closer than the bf16 block (a chain still rounding to bf16
    somewhere would not), and both are within a few bf16 roundings of it;
    every relation it writes is a half value.  Token rows agree with the
    full form bit for bit."""
    w, batch, seq, heads = _tiny_block(7, T=64, Dm=16, heads=2, F=12, batch=2)
    yb = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    yh, mid = orc.llama_block(**w, batch=batch, seq=seq, heads=heads, dtype="f16", return_intermediates=True)
    for k in ("h1", "qkv", "O", "x2", "h2", "f"):
        assert np.array_equal(mid[k], orc.round_f16(mid[k]))
    assert np.array_equal(yh, orc.round_f16(yh)) and not np.array_equal(yh, orc.round_bf16(yh))
    # the chain with no rounding: the same formulas with the identity as rounding
    saved = orc.round_bf16
    try:
        orc.round_bf16 = lambda v: np.asarray(v, dtype=np.float64)
        y0 = orc.llama_block(**w, batch=batch, seq=seq, heads=heads)
    finally:
        orc.round_bf16 = saved
    eb, eh = np.linalg.norm(yb - y0), np.linalg.norm(yh - y0)
    assert 3.0 * eh < eb <= 2.0 ** -5 * np.linalg.norm(y0)
    toks = [0, 5, seq - 1, seq + 3]
    yt = orc.llama_block_tokens(**w, batch=batch, seq=seq, heads=heads, tokens=toks, dtype="f16")
    assert np.array_equal(yt, yh[toks])


def test_gqa_block_equals_mha_block_on_expanded_weights(orc):
    """Grouped-query block (4 query heads over 2 key-value heads, section
    3.3): the same as the multi-head block whose W_k and W_v repeat each
    key-value head's columns for the query heads of its group -- bit for
    bit, since every output element is computed from the same values in the
    same order.  The token-sampled form agrees with the full form."""
    rng = np.random.default_rng(6)
    T, Dm, heads, kv, F, batch = 12, 16, 4, 2, 6, 2
    hd = Dm // heads
    r = lambda a: rng.standard_normal(a) * 0.5
    w = dict(x=orc.round_bf16(r((T, Dm))), g1=1 + 0.1 * r(Dm), w_qkv=r((Dm, Dm + 2 * kv * hd)), w_o=r((Dm, Dm)),
             g2=1 + 0.1 * r(Dm), w_gate=r((Dm, F)), w_up=r((Dm, F)), w_down=r((F, Dm)))
    y = orc.llama_block(**w, batch=batch, seq=T // batch, heads=heads, kv_heads=kv)
    wq, wk, wv = w["w_qkv"][:, :Dm], w["w_qkv"][:, Dm:Dm + kv * hd], w["w_qkv"][:, Dm + kv * hd:]
    grp = [h // (heads // kv) for h in range(heads)]
    expand = lambda m: np.concatenate([m[:, g * hd:(g + 1) * hd] for g in grp], axis=1)
    w_mha = dict(w, w_qkv=np.concatenate([wq, expand(wk), expand(wv)], axis=1))
    assert np.array_equal(y, orc.llama_block(**w_mha, batch=batch, seq=T // batch, heads=heads))
    toks = [0, 4, 5, 6, 11]
    yt = orc.llama_block_tokens(**w, batch=batch, seq=T // batch, heads=heads, tokens=toks, kv_heads=kv)
    assert np.array_equal(yt, y[toks])


def test_packed_attention_is_per_sequence_attention(orc):
    """Packed sequences (the pages' section 3.3): three sequences ending at 5,
    13 and 20 along one index.  Each query sees only its own sequence, so the
    packed result equals attention run on every sequence by itself -- causal
    and not, multi-head and grouped-query; one sequence is plain attention."""
    rng = np.random.default_rng(41)
    S, D, ends = 20, 8, [5, 13, 20]
    for H, HK in ((2, 2), (4, 2)):
        Q = rng.standard_normal((2, H, S, D))
        K, V = (rng.standard_normal((2, HK, S, D)) for _ in range(2))
        for causal in (True, False):
            got = orc.attention(Q, K, V, 0.6, causal, seq_ends=ends)
            for a, b in zip([0] + ends[:-1], ends):
                want = orc.attention(Q[:, :, a:b], K[:, :, a:b], V[:, :, a:b], 0.6, causal)
                np.testing.assert_allclose(got[:, :, a:b], want, rtol=1e-14, atol=1e-15)
            np.testing.assert_array_equal(orc.attention(Q, K, V, 0.6, causal, seq_ends=[S]),
                                          orc.attention(Q, K, V, 0.6, causal))
    with pytest.raises(ValueError):
        orc.attention(Q, K, V, 0.6, True, seq_ends=[5, 13])  # must end at S


def test_packed_tuple_counts(orc):
    """The pages' example: 4,096 positions holding sequences that end at
    1,024, 2,560 and 4,096.  Cut at every sequence end, only the three
    diagonal (query block, key block) cells share a sequence; cut at 1,024
    only, the two blocks hold no common sequence, so the off-diagonal cells
    drop too."""
    ends = [1024, 2560, 4096]
    sp = {"s": [0, 1024, 2560, 4096], "t": [0, 1024, 2560, 4096], "d": [0, 128]}
    for causal in (("s", "t"), None):
        rec, seg = orc.tuple_records("sdt", sp, "s", causal=causal, packed=("s", "t", ends))
        assert rec[:, [0, 2]].tolist() == [[0, 0], [1, 1], [2, 2]] and len(seg) - 1 == 3
    sp2 = {"s": [0, 1024, 4096], "t": [0, 1024, 4096], "d": [0, 128]}
    rec, _ = orc.tuple_records("sdt", sp2, "s", causal=None, packed=("s", "t", ends))
    assert rec[:, [0, 2]].tolist() == [[0, 0], [1, 1]]
    # without the packing predicate a causal cut keeps the lower triangle
    rec, _ = orc.tuple_records("sdt", sp, "s", causal=("s", "t"))
    assert rec.shape[0] == 6


# ---------------------------------------------------------------- IEEE half (fp16 relations)

def test_f16_known_encodings(orc):
    cases = {
        1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF,         # largest finite half
        65519.0: 0x7BFF, 65520.0: 0x7C00,                   # the tie at the top rounds to even: infinity
        2.0 ** -14: 0x0400, 2.0 ** -24: 0x0001,             # smallest normal, smallest subnormal
        2.0 ** -25: 0x0000, 3 * 2.0 ** -25: 0x0002,         # ties to even in the subnormal range
        1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02,  # ties to even at 1
        0.1: 0x2E66, -0.0: 0x8000,
    }
    xs = np.array(list(cases.keys()))
    got = orc.f64_to_f16(xs)
    assert [int(v) for v in got] == list(cases.values())
    assert orc.f64_to_f16(np.array([np.inf]))[0] == 0x7C00
    assert orc.f64_to_f16(np.array([np.nan]))[0] & 0x7FFF > 0x7C00


def test_f16_all_patterns_and_independent_route(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = orc.f16_to_f64(h)
    fin = np.isfinite(v)
    assert np.array_equal(orc.f64_to_f16(v[fin]), h[fin])          # every finite pattern round trips
    assert np.array_equal(v[fin], h[fin].view(np.float16).astype(np.float64))  # numpy's decode
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-6, 1e-3, 1.0, 1e3, 6e4)])
    with np.errstate(over="ignore"):  # the widest scale overflows to infinity on both routes
        assert np.array_equal(orc.f64_to_f16(x), x.astype(np.float16).view(np.uint16))  # numpy's RNE encode
