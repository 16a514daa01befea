"""Seeded random decompositions on the GPU, every output element against the
oracle.

The hand-written cases in test_gpu_ops.py pick the shapes a reader can
check; these draw them: random extents, interval counts and cut positions
for every letter; every operand layout of a contraction (with a batch letter
too) in bf16, fp16 and fp32; causal and non-causal attention with multi-head
and grouped-query specs in bf16 and fp16; packed sequences with random ends,
cut at a random subset of them; RMSNorm and the 1:1 joins over random
blockings; repartitions through random reshape-and-permute views (bit-exact).  The draws are fixed by the case number, so a failing case is
rerun by its id.  Bars as everywhere: fp32 contractions infinity-norm
relative <= 1e-5; 16-bit relations (fp32 accumulation) relative Frobenius
<= 2e-3 against the oracle rounded to the output format, and for the
contractions, RMSNorm and the 1:1 joins nearly every element equal to it."""
import numpy as np
import pytest

from gpu_helpers import record, rel_frobenius, rel_inf
from test_gpu_ops import _repart_case, _run
from tensor_relational_join_amd import synth

pytestmark = pytest.mark.gpu
TOL16 = 2e-3
TOL32 = 1e-5


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available()
    from tensor_relational_join_amd import device

    return device


def _cuts(rng, n, qmax, step):
    """Split points of [0, n) into 1..qmax intervals, cut at multiples of `step`."""
    inner = [c for c in range(step, n, step)]
    q = int(rng.integers(1, qmax + 1))
    q = min(q, len(inner) + 1)
    picked = sorted(rng.choice(inner, size=q - 1, replace=False).tolist()) if q > 1 else []
    return [0] + picked + [n]


CONTRACT_LAYOUTS = ["ij,jk->ik", "ij,kj->ik", "ji,jk->ik", "ji,kj->ik", "bij,bjk->bik", "bji,bkj->bik"]


def _contract_case(case):
    rng = np.random.default_rng(1000 + case)
    einsum = CONTRACT_LAYOUTS[case % len(CONTRACT_LAYOUTS)]
    dt = ["bf16", "bf16", "f16", "f32"][int(rng.integers(0, 4))]
    ext = {c: 8 * int(rng.integers(1, 76)) for c in "ijk"}  # multiples of 8 up to 600
    ext["b"] = int(rng.integers(1, 4))
    sp = {c: _cuts(rng, ext[c], 3, 8) for c in "ijk"}
    sp["b"] = _cuts(rng, ext["b"], 3, 1)
    return einsum, dt, {c: sp[c] for c in set(einsum) - {",", "-", ">"}}


@pytest.mark.parametrize("case", range(48))
def test_random_contraction(dev, orc, case):
    from tensor_relational_join_amd.binding import JA_BF16, JA_F16, JA_F32

    einsum, dt, sp = _contract_case(case)
    print("case", case, einsum, dt, sp, flush=True)
    lhs, out = einsum.split("->")
    shapes = [tuple(sp[c][-1] for c in s) for s in lhs.split(",")]
    if dt == "f32":
        rng = np.random.default_rng(2000 + case)
        X, W = (rng.uniform(-1.0, 1.0, size=s).astype(np.float32) for s in shapes)
        got, o, _ = _run(dev, orc, einsum, "contract", sp, [X, W], in_dtypes=[JA_F32, JA_F32], out_dtype=JA_F32)
        o.close()
        want = orc.einsum(einsum, X.astype(np.float64), W.astype(np.float64))
        err = rel_inf(got, want)
        record("random_contraction", case=case, dtype=dt, rel_inf=err)
        assert err <= TOL32, (case, err)
        return
    gen, dec, rnd, code = ((synth.normal_bf16, orc.bf16_to_f64, orc.round_bf16, JA_BF16) if dt == "bf16" else
                           (synth.normal_f16, orc.f16_to_f64, orc.round_f16, JA_F16))
    X = gen(3000 + case, 0, shapes[0])
    W = gen(3000 + case, 1, shapes[1], std=0.05)
    got, o, _ = _run(dev, orc, einsum, "contract", sp, [X, W], in_dtypes=[code, code], out_dtype=code)
    o.close()
    want = rnd(orc.einsum(einsum, dec(X), dec(W)))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("random_contraction", case=case, dtype=dt, rel_frobenius=err, equal_fraction=eq)
    assert err <= TOL16, (case, err)
    assert eq > 0.9, (case, eq)


def _attention_case(case):
    rng = np.random.default_rng(5000 + case)
    gqa = case % 3 == 2
    causal = bool(case % 2 == 0)
    dt = "f16" if case % 4 == 3 else "bf16"
    Bn = int(rng.integers(1, 3))
    S = int(rng.integers(1, 421))
    T = S if causal else int(rng.integers(1, 421))
    sp = {"b": _cuts(rng, Bn, 2, 1), "s": _cuts(rng, S, 4, 1), "t": _cuts(rng, T, 4, 1), "d": [0, 128]}
    if gqa:
        G, R = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        sp.update(g=_cuts(rng, G, 2, 1), r=_cuts(rng, R, 3, 1))
        return "bgrsd,bgtd,bgtd->bgrsd", causal, dt, sp, (Bn, G, R, S, T)
    H = int(rng.integers(1, 4))
    sp["h"] = _cuts(rng, H, 3, 1)
    return "bhsd,bhtd,bhtd->bhsd", causal, dt, sp, (Bn, H, 1, S, T)


@pytest.mark.parametrize("case", range(24))
def test_random_attention(dev, orc, case):
    from tensor_relational_join_amd.binding import JA_BF16, JA_F16

    einsum, causal, dt, sp, (Bn, G, R, S, T) = _attention_case(case)
    print("case", case, einsum, "causal" if causal else "non-causal", dt, sp, flush=True)
    gen, dec, rnd, code = ((synth.normal_bf16, orc.bf16_to_f64, orc.round_bf16, JA_BF16) if dt == "bf16" else
                           (synth.normal_f16, orc.f16_to_f64, orc.round_f16, JA_F16))
    qshape = (Bn, G, R, S, 128) if einsum.startswith("bgr") else (Bn, G, S, 128)
    Q = gen(6000 + case, 0, qshape)
    K = gen(6000 + case, 1, (Bn, G, T, 128))
    V = gen(6000 + case, 2, (Bn, G, T, 128))
    got, o, _ = _run(dev, orc, einsum, "attention", sp, [Q, K, V], params="causal=s,t" if causal else "",
                     in_dtypes=[code] * 3, out_dtype=code)
    o.close()
    want = orc.attention(dec(Q).reshape(Bn, G * R, S, 128), dec(K), dec(V), 1.0 / np.sqrt(128.0), causal)
    err = rel_frobenius(got, rnd(want).reshape(got.shape))
    record("random_attention", case=case, dtype=dt, causal=causal, rel_frobenius=err)
    assert err <= TOL16, (case, err)


@pytest.mark.parametrize("case", range(12))
def test_random_packed_attention(dev, orc, case):
    """Sequences packed along s and t with random ends; the decomposition cuts
    s and t at a random subset of the ends (the only legal cuts)."""
    rng = np.random.default_rng(7000 + case)
    S = int(rng.integers(2, 401))
    n = int(rng.integers(1, min(6, S) + 1))
    ends = sorted(rng.choice(np.arange(1, S), size=n - 1, replace=False).tolist()) + [S] if n > 1 else [S]
    inner = ends[:-1]
    k = int(rng.integers(0, len(inner) + 1))
    cuts = [0] + sorted(rng.choice(inner, size=k, replace=False).tolist() if k else []) + [S]
    HK, R = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal = bool(case % 2 == 0)
    print("case", case, "S", S, "ends", ends, "cuts", cuts, "heads", HK * R, "/", HK,
          "causal" if causal else "non-causal", flush=True)
    sp = {"b": [0, 1], "g": _cuts(rng, HK, 2, 1), "r": [0, R], "s": cuts, "t": cuts, "d": [0, 128]}
    Q = synth.normal_bf16(7500 + case, 0, (1, HK, R, S, 128))
    K = synth.normal_bf16(7500 + case, 1, (1, HK, S, 128))
    V = synth.normal_bf16(7500 + case, 2, (1, HK, S, 128))
    params = "packed=" + ",".join(map(str, ends)) + (";causal=s,t" if causal else "")
    got, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V], params=params)
    o.close()
    want = orc.attention(orc.bf16_to_f64(Q).reshape(1, HK * R, S, 128), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                         1.0 / np.sqrt(128.0), causal, seq_ends=ends)
    err = rel_frobenius(got.reshape(1, HK * R, S, 128), orc.round_bf16(want))
    record("random_packed_attention", case=case, rel_frobenius=err)
    assert np.isfinite(got).all()
    assert err <= TOL16, (case, err)


@pytest.mark.parametrize("case", range(12))
def test_random_rmsnorm(dev, orc, case):
    rng = np.random.default_rng(8000 + case)
    R, D = int(rng.integers(1, 300)), int(rng.integers(1, 9)) * 128 * int(rng.integers(1, 3))
    sp = {"r": _cuts(rng, R, 3, 1), "d": _cuts(rng, D, 4, int(rng.choice([1, 8, 64])))}
    print("case", case, "R", R, "D", D, sp, flush=True)
    x = synth.normal_bf16(8500 + case, 0, (R, D))
    g = synth.normal_bf16(8500 + case, 1, (D,), mean=1.0, std=0.1)
    got, o, _ = _run(dev, orc, "rd,d->rd", "rmsnorm", sp, [x, g], params="eps=1e-6")
    o.close()
    want = orc.round_bf16(orc.rmsnorm(orc.bf16_to_f64(x), orc.bf16_to_f64(g), 1e-6))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("random_rmsnorm", case=case, rel_frobenius=err, equal_fraction=eq)
    assert err <= TOL16, (case, err)
    assert eq > 0.99, (case, eq)


@pytest.mark.parametrize("case", range(12))
def test_random_one_to_one_joins(dev, orc, case):
    rng = np.random.default_rng(9000 + case)
    op = "swiglu" if case % 2 == 0 else "add"
    R, F = int(rng.integers(1, 200)), int(rng.integers(1, 700))
    sp = {"r": _cuts(rng, R, 3, 1), "f": _cuts(rng, F, 4, 1)}
    print("case", case, op, "R", R, "F", F, sp, flush=True)
    a = synth.normal_bf16(9500 + case, 0, (R, F))
    b = synth.normal_bf16(9500 + case, 1, (R, F))
    got, o, _ = _run(dev, orc, "rf,rf->rf", op, sp, [a, b])
    o.close()
    af, bf = orc.bf16_to_f64(a), orc.bf16_to_f64(b)
    want = orc.round_bf16(orc.swiglu(af, bf) if op == "swiglu" else orc.add(af, bf))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("random_one_to_one_joins", case=case, op=op, rel_frobenius=err, equal_fraction=eq)
    assert err <= TOL16, (case, err)
    assert eq > 0.99, (case, eq)


def _group(rng, factors):
    """Consecutive factors merged into dimensions at random."""
    dims, cur = [], 1
    for i, f in enumerate(factors):
        cur *= f
        if i == len(factors) - 1 or rng.random() < 0.5:
            dims.append(cur)
            cur = 1
    return tuple(dims)


@pytest.mark.parametrize("case", range(16))
def test_random_view_repartition(dev, orc, case):
    """A tensor re-indexed through a view: its shape and the destination's
    are random groupings of the same factors, the view permutes the factors,
    and both sides are blocked at random; every element bit for bit."""
    rng = np.random.default_rng(10000 + case)
    factors = [int(x) for x in rng.integers(1, 25 if case % 4 else 9, int(rng.integers(2, 5)))]
    perm = [int(x) for x in rng.permutation(len(factors))]
    src = _group(rng, factors)
    dst = _group(rng, [factors[p] for p in perm])
    src_sp = [_cuts(rng, n, 3, 1) for n in src]
    dst_sp = [_cuts(rng, n, 3, 1) for n in dst]
    print("case", case, "factors", factors, "perm", perm, "src", src, src_sp, "dst", dst, dst_sp, flush=True)
    _repart_case(dev, orc, src, src_sp, dst, dst_sp, vshape=tuple(factors), perm=perm,
                 dtype="bf16" if case % 2 else "f32", seed=case)
