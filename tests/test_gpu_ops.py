"""GPU parity of every join-agg operator against the CPU oracle, through the
C ABI.  Inputs are seeded synthetic tensors packed into relations by the
oracle's own layout code; outputs are unpacked the same way and compared
with the oracle's dense result (rounded to bf16 where the output is bf16).

Bars: fp32 -> infinity-norm relative error <= 1e-5; bf16 inputs with fp32
accumulation -> relative Frobenius error <= 2e-3; tuple lists and
repartitions -> bit-exact."""
import itertools

import numpy as np
import pytest

from gpu_helpers import bf16_bits, f32_host, record, rel_frobenius, rel_inf, to_dev_bf16, to_dev_f16, to_dev_f32
from tensor_relational_join_amd import synth

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5
BF16_TOL = 2e-3


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


def _run(dev, orc, einsum, op, splits, dense_inputs, params="", in_dtypes=None, out_dtype=None):
    """Pack inputs with the oracle's layout code, run the op through the C ABI,
    unpack the output relation with the oracle's layout code."""
    import torch

    from tensor_relational_join_amd.binding import JA_BF16, JA_F16, JA_F32

    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    in_dtypes = in_dtypes or [JA_BF16] * len(ins)
    out_dtype = JA_BF16 if out_dtype is None else out_dtype
    o = dev.Op(einsum, op, splits, params, in_dtypes, out_dtype)
    try:
        dev_ins = []
        for s, x, dt in zip(ins, dense_inputs, in_dtypes):
            rel = orc.Relation([splits[c][-1] for c in s], [splits[c] for c in s])
            flat = rel.pack(x)
            dev_ins.append(to_dev_bf16(flat) if dt == JA_BF16 else to_dev_f16(flat) if dt == JA_F16 else
                           to_dev_f32(flat))
        out_t = dev.alloc(o.out_rel)
        o.run(dev_ins, out_t)
        torch.cuda.synchronize()
        orel = orc.Relation([splits[c][-1] for c in out], [splits[c] for c in out])
        host = bf16_bits(out_t) if out_dtype in (JA_BF16, JA_F16) else f32_host(out_t)
        res = orel.unpack(host)
        if out_dtype == JA_BF16:
            res = orc.bf16_to_f64(res)
        elif out_dtype == JA_F16:
            res = orc.f16_to_f64(res)
        return res.astype(np.float64), o, dev_ins
    except Exception:
        o.close()
        raise


# ------------------------------------------------------------------ contraction, fp32 (2x2x2, 64^3)

def test_matmul_fp32_2x2x2(dev, orc):
    from tensor_relational_join_amd.binding import JA_F32

    A = synth.uniform(1, 0, (64, 64))
    Bm = synth.uniform(1, 1, (64, 64))
    sp = {c: _eq(64, 2) for c in "ijk"}
    got, o, ins = _run(dev, orc, "ij,jk->ik", "contract", sp, [A, Bm], in_dtypes=[JA_F32, JA_F32], out_dtype=JA_F32)
    try:
        assert o.tuples()[0].shape[0] == 8
        want = orc.einsum("ij,jk->ik", A, Bm)
        assert rel_inf(got, want) <= FP32_TOL
        # the scalar relational join-agg of the same inputs agrees too
        assert rel_inf(got, orc.brute_force_einsum("ij,jk->ik", A, Bm)) <= FP32_TOL
        # unfused path: per-tuple partials, then the SUM aggregation
        import torch

        part = o.partial_buffer()
        o.kernel(ins, part)
        out2 = torch.empty(64 * 64, dtype=torch.float32, device="cuda")
        o.agg(part, out2)
        torch.cuda.synchronize()
        orel = orc.Relation((64, 64), [sp["i"], sp["k"]])
        got2 = orel.unpack(f32_host(out2)).astype(np.float64)
        assert rel_inf(got2, want) <= FP32_TOL
        # each partial is one tuple's block product
        rec, seg = o.tuples()
        p = f32_host(part)
        for t, r in enumerate(rec.tolist()):
            iv = {c: (sp[c][r[o.letters.index(c)]], sp[c][r[o.letters.index(c)] + 1]) for c in "ijk"}
            blk = orc.einsum("ij,jk->ik", A[iv["i"][0]:iv["i"][1], iv["j"][0]:iv["j"][1]],
                             Bm[iv["j"][0]:iv["j"][1], iv["k"][0]:iv["k"][1]])
            assert rel_inf(p[t * 1024:(t + 1) * 1024].reshape(32, 32), blk) <= FP32_TOL
    finally:
        o.close()


def test_one_cell_blocks_fp32(dev, orc):
    """The degenerate decomposition: every interval one element long, so every
    tuple joins two scalars and every segment sums j of them -- the scalar
    relational join-agg of the paper's section 1, run on the GPU.  Small
    integers keep every product and sum exact, so the result must equal the
    brute-force join bit for bit, fused and unfused."""
    import torch

    from tensor_relational_join_amd.binding import JA_F32

    rng = np.random.default_rng(7)
    I, J, K = 5, 4, 3
    A = rng.integers(-3, 4, (I, J)).astype(np.float64)
    Bm = rng.integers(-3, 4, (J, K)).astype(np.float64)
    sp = {"i": list(range(I + 1)), "j": list(range(J + 1)), "k": list(range(K + 1))}
    got, o, ins = _run(dev, orc, "ij,jk->ik", "contract", sp, [A, Bm], in_dtypes=[JA_F32, JA_F32], out_dtype=JA_F32)
    try:
        rec, seg = o.tuples()
        assert rec.shape[0] == I * J * K and len(seg) - 1 == I * K
        want = orc.brute_force_einsum("ij,jk->ik", A, Bm)
        assert np.array_equal(got, want)
        part = o.partial_buffer()
        o.kernel(ins, part)
        out2 = torch.empty(I * K, dtype=torch.float32, device="cuda")
        o.agg(part, out2)
        torch.cuda.synchronize()
        got2 = orc.Relation((I, K), [sp["i"], sp["k"]]).unpack(f32_host(out2)).astype(np.float64)
        assert np.array_equal(got2, want)
        # each one-element partial is the product of its tuple's two cells
        p = f32_host(part)
        for t, r in enumerate(rec.tolist()):
            i, j, k = (r[o.letters.index(c)] for c in "ijk")
            assert p[t] == A[i, j] * Bm[j, k]
    finally:
        o.close()


@pytest.mark.parametrize("case", ["f32_ragged", "bf16"])
def test_aggregation_of_host_partials(dev, orc, case):
    """ja_agg alone, on fp32 partial blocks drawn on the host and laid out as
    the unfused path lays them out (one block per tuple, in tuple order).
    The fp32 case has block sizes that are not multiples of 4, so some
    segments fold element by element and others in 16-byte vectors; the bf16
    case writes packed halves.  SUM against the fold written out in float64,
    MAX exactly."""
    import torch

    from tensor_relational_join_amd.binding import JA_AGG_MAX, JA_AGG_SUM, JA_BF16, JA_F32

    if case == "f32_ragged":
        sp = {"i": [0, 37, 100, 1125], "j": [0, 40, 72, 136], "k": [0, 29, 90, 2137]}
        dt = JA_F32
    else:
        sp = {"i": [0, 40, 104, 1128], "j": [0, 40, 72, 136], "k": [0, 32, 96, 2144]}
        dt = JA_BF16
    o = dev.Op("ij,jk->ik", "contract", sp, "", [dt, dt], dt)
    try:
        rec, seg = o.tuples()
        li, lk = o.letters.index("i"), o.letters.index("k")
        sizes = [(sp["i"][r[li] + 1] - sp["i"][r[li]]) * (sp["k"][r[lk] + 1] - sp["k"][r[lk]]) for r in rec.tolist()]
        offs = np.concatenate([[0], np.cumsum(sizes)])
        rng = np.random.default_rng(11)
        part = rng.standard_normal(int(offs[-1])).astype(np.float32)
        part_dev = torch.from_numpy(part).cuda()
        orel = orc.Relation((sp["i"][-1], sp["k"][-1]), [sp["i"], sp["k"]])
        for op in (JA_AGG_SUM, JA_AGG_MAX):
            want = np.zeros((sp["i"][-1], sp["k"][-1]))
            for sgi in range(len(seg) - 1):
                ts = range(int(seg[sgi]), int(seg[sgi + 1]))
                r = rec[ts[0]]
                i0, i1 = sp["i"][r[li]], sp["i"][r[li] + 1]
                k0, k1 = sp["k"][r[lk]], sp["k"][r[lk] + 1]
                blocks = [part[offs[t]:offs[t + 1]].astype(np.float64).reshape(i1 - i0, k1 - k0) for t in ts]
                fold = blocks[0].copy()
                for b in blocks[1:]:
                    fold = fold + b if op == JA_AGG_SUM else np.maximum(fold, b)
                want[i0:i1, k0:k1] = fold
            out = dev.alloc(o.out_rel)
            o.agg(part_dev, out, op=op)
            torch.cuda.synchronize()
            if dt == JA_F32:
                got = orel.unpack(f32_host(out)).astype(np.float64)
                if op == JA_AGG_MAX:
                    assert np.array_equal(got, want)
                else:
                    assert rel_inf(got, want) <= FP32_TOL
            else:
                got = orc.bf16_to_f64(orel.unpack(bf16_bits(out)))
                want_b = orc.round_bf16(want)
                if op == JA_AGG_MAX:
                    assert np.array_equal(got, want_b)
                else:
                    assert rel_frobenius(got, want_b) <= BF16_TOL
                    assert np.mean(got == want_b) > 0.99
    finally:
        o.close()


def test_max_aggregation_fp32(dev, orc):
    import torch

    from tensor_relational_join_amd.binding import JA_AGG_MAX, JA_F32

    A = synth.uniform(2, 0, (40, 48))
    Bm = synth.uniform(2, 1, (48, 24))
    sp = {"i": [0, 40], "j": [0, 16, 24, 48], "k": [0, 24]}
    got, o, ins = _run(dev, orc, "ij,jk->ik", "contract", sp, [A, Bm], in_dtypes=[JA_F32, JA_F32], out_dtype=JA_F32)
    try:
        part = o.partial_buffer()
        o.kernel(ins, part)
        out = torch.empty(40 * 24, dtype=torch.float32, device="cuda")
        o.agg(part, out, op=JA_AGG_MAX)
        torch.cuda.synchronize()
        want = np.max([orc.einsum("ij,jk->ik", A[:, a:b], Bm[a:b]) for a, b in [(0, 16), (16, 24), (24, 48)]], axis=0)
        assert rel_inf(f32_host(out).reshape(40, 24), want) <= FP32_TOL
    finally:
        o.close()


# ------------------------------------------------------------------ contraction, bf16 MFMA

BF16_CASES = [
    # einsum, splits, shapes (per operand letters)
    ("ij,jk->ik", {"i": [0, 100, 300], "j": [0, 64, 256], "k": [0, 136, 264]}),
    ("ij,jk->ik", {"i": [0, 129], "j": [0, 8, 200, 392], "k": [0, 8, 128, 136]}),
    ("ij,kj->ik", {"i": [0, 77, 200], "j": [0, 96, 320], "k": [0, 50, 130]}),
    ("ji,jk->ik", {"i": [0, 64, 200], "j": [0, 160, 320], "k": [0, 72, 144]}),
    ("ji,kj->ik", {"i": [0, 136], "j": [0, 64, 128], "k": [0, 40, 96]}),
    ("bij,bjk->bik", {"b": [0, 2, 3], "i": [0, 70, 130], "j": [0, 64, 192], "k": [0, 80, 160]}),
    # a segment shorter than the load pipeline: one 32-wide stage, then two
    ("ij,jk->ik", {"i": [0, 64], "j": [0, 24], "k": [0, 40, 80]}),
    ("ij,kj->ik", {"i": [0, 300], "j": [0, 40], "k": [0, 264]}),
    # several tiles with ragged tails and uneven tuples inside a segment
    ("ij,jk->ik", {"i": [0, 520], "j": [0, 200, 336, 432], "k": [0, 776]}),
    ("ji,jk->ik", {"i": [0, 264, 520], "j": [0, 96, 328], "k": [0, 256, 264]}),
]


@pytest.mark.parametrize("einsum,sp", BF16_CASES)
def test_contract_bf16_ragged_and_layouts(dev, orc, einsum, sp):
    lhs, out = einsum.split("->")
    shapes = [tuple(sp[c][-1] for c in s) for s in lhs.split(",")]
    X = synth.normal_bf16(3, 0, shapes[0])
    W = synth.normal_bf16(3, 1, shapes[1], std=0.02)
    got, o, _ = _run(dev, orc, einsum, "contract", sp, [X, W])
    o.close()
    want = orc.round_bf16(orc.einsum(einsum, orc.bf16_to_f64(X), orc.bf16_to_f64(W)))
    assert rel_frobenius(got, want) <= BF16_TOL
    # the bf16 outputs are the correctly rounded fp32 sums: nearly all equal the rounded oracle
    assert np.mean(got == want) > 0.95


def test_contract_bf16_f32_output_and_determinism(dev, orc):
    import torch

    from tensor_relational_join_amd.binding import JA_BF16, JA_F32

    sp = {"i": [0, 256, 384], "j": [0, 512, 1024], "k": [0, 128, 520]}
    X = synth.normal_bf16(4, 0, (384, 1024))
    W = synth.normal_bf16(4, 1, (1024, 520), std=0.02)
    got, o, ins = _run(dev, orc, "ij,jk->ik", "contract", sp, [X, W], out_dtype=JA_F32)
    try:
        want = orc.einsum("ij,jk->ik", orc.bf16_to_f64(X), orc.bf16_to_f64(W))
        assert rel_inf(got, want) <= 1e-5  # fp32 accumulation of exact bf16 products
        a = dev.alloc(o.out_rel)
        b = dev.alloc(o.out_rel)
        o.run(ins, a)
        o.run(ins, b)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))  # bitwise run-to-run
    finally:
        o.close()
    assert JA_BF16 != JA_F32


def test_ffn_contraction_full_size(dev, orc):
    """b=2048, d=4096, f=11008 split 2 x 4 x 4: 32 tuples, 8 segments of 4,
    352 output tiles (a full round on 256 compute units and a half-height
    last round); every output element against the oracle."""
    sp = {"b": _eq(2048, 2), "d": _eq(4096, 4), "f": _eq(11008, 4)}
    X = synth.normal_bf16(2, 0, (2048, 4096))
    W = synth.normal_bf16(2, 1, (4096, 11008), std=0.02)
    got, o, _ = _run(dev, orc, "bd,df->bf", "contract", sp, [X, W])
    rec, seg = o.tuples()
    o.close()
    assert rec.shape[0] == 32 and len(seg) - 1 == 8
    want = orc.round_bf16(orc.einsum("bd,df->bf", orc.bf16_to_f64(X), orc.bf16_to_f64(W)))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("ffn_contraction_full_size", rel_frobenius=err, equal_fraction=eq)
    assert err <= BF16_TOL
    assert eq > 0.95


def test_contraction_persistent_multi_tile_walk(dev, orc):
    """One segment of 868 output tiles of 256 x 256 (ragged in both
    directions, 28 x 31): the persistent kernel's 256 workgroups walk three
    tiles each (each loads its next tile's first stage while the current
    tile's results leave) and the last 100 tiles run as 200 half-height tiles
    in a second launch.  868 is a multiple of neither 8 nor 256, so the XCD
    deal is uneven.  K = 136 in two tuples (64 and 72: a ragged last stage),
    every output element against the oracle."""
    M, N = 7000, 7800
    sp = {"i": [0, M], "j": [0, 64, 136], "k": [0, N]}
    X = synth.normal_bf16(9, 0, (M, 136))
    W = synth.normal_bf16(9, 1, (136, N), std=0.1)
    got, o, _ = _run(dev, orc, "ij,jk->ik", "contract", sp, [X, W])
    o.close()
    assert (-(-M // 256)) * (-(-N // 256)) == 868
    want = orc.round_bf16(orc.einsum("ij,jk->ik", orc.bf16_to_f64(X), orc.bf16_to_f64(W)))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("contraction_persistent_multi_tile_walk", rel_frobenius=err, equal_fraction=eq)
    assert err <= BF16_TOL
    assert eq > 0.95


# Contraction operands blocked coarser than the decomposition: each tuple reads
# a sub-box of its operand block in place (the block's row length as leading
# dimension), fused and through per-tuple partials and their SUM.
COARSE_CASES = [
    # (einsum, op, decomposition, the inputs' own blockings)
    ("ij,jk->ik", "contract", {"i": [0, 256, 520], "j": [0, 64, 136, 200, 256], "k": [0, 264, 520]},
     [{"j": [0, 136, 256]}, {"j": [0, 256], "k": [0, 520]}]),
    ("ji,kj->ik", "contract", {"i": [0, 136, 264], "j": [0, 96, 160, 256], "k": [0, 128, 392]},
     [{"j": [0, 256], "i": [0, 264]}, {"j": [0, 160, 256]}]),
    ("ij,jk,ik->ik", "contract_add", {"i": [0, 256, 520], "j": [0, 64, 136, 200, 256], "k": [0, 264, 520]},
     [{"j": [0, 256]}, None, None]),
]


@pytest.mark.parametrize("einsum,op,sp,own", COARSE_CASES)
def test_contraction_operands_blocked_coarser(dev, orc, einsum, op, sp, own):
    import torch

    from tensor_relational_join_amd.binding import JA_BF16

    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    shapes = [tuple(sp[c][-1] for c in x) for x in ins]
    dense = [synth.normal_bf16(43, i, shp, std=0.05 if i == 1 else 1.0) for i, shp in enumerate(shapes)]
    o = dev.Op(einsum, op, sp, "", [JA_BF16] * len(ins), JA_BF16, in_splits=own)
    try:
        dev_ins = [to_dev_bf16(orc.Relation([sp[c][-1] for c in x], [(blk or {}).get(c, sp[c]) for c in x]).pack(v))
                   for x, v, blk in zip(ins, dense, own)]
        orel = orc.Relation([sp[c][-1] for c in out], [sp[c] for c in out])
        out_t = dev.alloc(o.out_rel)
        o.run(dev_ins, out_t)
        torch.cuda.synchronize()
        got = orc.bf16_to_f64(orel.unpack(bf16_bits(out_t)))
        unfused = None
        if op == "contract":  # per-tuple partials over the same sub-boxes, then the SUM
            part = o.partial_buffer()
            o.kernel(dev_ins, part)
            out2 = dev.alloc(o.out_rel)
            o.agg(part, out2)
            torch.cuda.synchronize()
            unfused = orc.bf16_to_f64(orel.unpack(bf16_bits(out2)))
    finally:
        o.close()
    w = [orc.bf16_to_f64(x) for x in dense]
    plain = "%s,%s->%s" % (ins[0], ins[1], out)
    want = orc.round_bf16(orc.contract_residual(plain, *w) if op == "contract_add" else orc.einsum(plain, w[0], w[1]))
    assert rel_frobenius(got, want) <= BF16_TOL
    assert np.mean(got == want) > 0.95
    if unfused is not None:
        assert rel_frobenius(unfused, want) <= BF16_TOL


# ------------------------------------------------------------------ attention

ATT_CASES = [
    ((1, 2, 384, 384), {"s": _eq(384, 3), "t": _eq(384, 3)}, True),
    ((2, 1, 256, 256), {"s": [0, 256], "t": [0, 256]}, True),
    ((1, 2, 300, 300), {"s": [0, 100, 300], "t": [0, 200, 300]}, True),     # uneven, ragged tiles
    ((1, 2, 256, 384), {"s": [0, 128, 256], "t": [0, 64, 384]}, False),     # non-causal, S != T
    ((2, 3, 200, 200), {"s": [0, 72, 200], "t": [0, 130, 200]}, True),
]


@pytest.mark.parametrize("shape,sst,causal", ATT_CASES)
def test_attention_small(dev, orc, shape, sst, causal):
    Bn, H, S, T = shape
    sp = {"b": _eq(Bn, Bn), "h": _eq(H, H), "s": sst["s"], "t": sst["t"], "d": [0, 128]}
    Q = synth.normal_bf16(5, 0, (Bn, H, S, 128))
    K = synth.normal_bf16(5, 1, (Bn, H, T, 128))
    V = synth.normal_bf16(5, 2, (Bn, H, T, 128))
    params = "causal=s,t" if causal else ""
    got, o, _ = _run(dev, orc, "bhsd,bhtd,bhtd->bhsd", "attention", sp, [Q, K, V], params=params)
    o.close()
    want = orc.round_bf16(orc.attention(orc.bf16_to_f64(Q), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                                        1.0 / np.sqrt(128.0), causal))
    assert rel_frobenius(got, want) <= BF16_TOL


def test_attention_full_size(dev, orc):
    """Q, K, V [4, 32, 2048, 128], 128-blocks on s and t, causal: 17,408
    tuples; every output row against the oracle's two-pass softmax."""
    Bn, H, S = 4, 32, 2048
    sp = {"b": _eq(Bn, Bn), "h": _eq(H, H), "s": _eq(S, 16), "t": _eq(S, 16), "d": [0, 128]}
    Q = synth.normal_bf16(3, 0, (Bn, H, S, 128))
    K = synth.normal_bf16(3, 1, (Bn, H, S, 128))
    V = synth.normal_bf16(3, 2, (Bn, H, S, 128))
    got, o, _ = _run(dev, orc, "bhsd,bhtd,bhtd->bhsd", "attention", sp, [Q, K, V], params="causal=s,t")
    rec, seg = o.tuples()
    o.close()
    assert rec.shape[0] == 17408 and len(seg) - 1 == 2048
    want = orc.round_bf16(orc.attention(orc.bf16_to_f64(Q), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                                        1.0 / np.sqrt(128.0), True))
    err, eq = rel_frobenius(got, want), float(np.mean(got == want))
    record("attention_full_size", rel_frobenius=err, equal_fraction=eq)
    assert err <= BF16_TOL


def test_attention_bf16_values_beyond_the_fp16_range(dev, orc):
    """bf16 V holding values far outside IEEE half's range: one head of
    1e5 .. 1e6, one of 1e-7, one ordinary, one whose keys alternate between
    the two extremes.  The kernel rounds V to fp16 for the P V product, so
    without its power-of-two V scale the first head would overflow to inf and
    the second would flush to zero.  Each head on its own meets the bar."""
    Bn, H, S = 1, 4, 384
    sp = {"b": [0, 1], "h": _eq(H, H), "s": _eq(S, 3), "t": _eq(S, 3), "d": [0, 128]}
    Q = synth.normal_bf16(17, 0, (Bn, H, S, 128))
    K = synth.normal_bf16(17, 1, (Bn, H, S, 128))
    base = orc.bf16_to_f64(synth.normal_bf16(17, 2, (Bn, H, S, 128)))
    mag = np.ones((Bn, H, S, 1))
    mag[:, 0] = 10.0 ** (5.0 + np.linspace(0.0, 1.0, S))[:, None]
    mag[:, 1] = 1e-7
    mag[:, 3, 0::2] = 1e6
    mag[:, 3, 1::2] = 1e-7
    V = orc.f64_to_bf16(base * mag)
    for causal in (True, False):
        got, o, _ = _run(dev, orc, "bhsd,bhtd,bhtd->bhsd", "attention", sp, [Q, K, V],
                         params="causal=s,t" if causal else "")
        o.close()
        want = orc.round_bf16(orc.attention(orc.bf16_to_f64(Q), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                                            1.0 / np.sqrt(128.0), causal))
        assert np.isfinite(got).all()
        errs = [rel_frobenius(got[:, h], want[:, h]) for h in range(H)]
        record("attention_bf16_values_beyond_the_fp16_range", causal=causal, per_head=errs)
        assert max(errs) <= BF16_TOL, errs


# ------------------------------------------------------------------ token-major attention

TOKEN_MAJOR_CASES = [
    # (einsum, Q shape, K shape, splits, causal): batch-head letters after the position letter, so a
    # block holds whole token rows of several heads
    ("bshd,bthd,bthd->bshd", (2, 384, 4, 128), (2, 384, 4, 128),
     {"b": [0, 1, 2], "s": _eq(384, 3), "t": _eq(384, 3), "h": [0, 4], "d": [0, 128]}, True),
    ("bshd,bthd,bthd->bshd", (1, 300, 3, 128), (1, 300, 3, 128),                  # heads cut 1 + 2, ragged tiles
     {"b": [0, 1], "s": [0, 100, 300], "t": [0, 200, 300], "h": [0, 1, 3], "d": [0, 128]}, True),
    ("bshd,bthd,bthd->bshd", (1, 256, 2, 128), (1, 384, 2, 128),                  # non-causal, S != T
     {"b": [0, 1], "s": [0, 128, 256], "t": [0, 64, 384], "h": [0, 2], "d": [0, 128]}, False),
    ("bsgrd,btgd,btgd->bsgrd", (1, 384, 2, 3, 128), (1, 384, 2, 128),             # grouped-query, r cut 1 + 2
     {"b": [0, 1], "s": _eq(384, 3), "t": _eq(384, 3), "g": [0, 2], "r": [0, 1, 3], "d": [0, 128]}, True),
]


def _heads_first(x):
    """[b, pos, heads..., d] -> [b, prod(heads), pos, d]"""
    x = np.moveaxis(x, 1, -2)
    return x.reshape(x.shape[0], -1, x.shape[-2], x.shape[-1])


@pytest.mark.parametrize("einsum,qshape,kshape,sp,causal", TOKEN_MAJOR_CASES)
def test_attention_token_major(dev, orc, einsum, qshape, kshape, sp, causal):
    """Q, K, V and O token-major (the projections' own layout): against the
    oracle's attention on the same values head-major, and bit for bit against
    the kernel on the head-major relations of the same values."""
    Q = synth.normal_bf16(23, 0, qshape)
    K = synth.normal_bf16(23, 1, kshape)
    V = synth.normal_bf16(23, 2, kshape)
    params = "causal=s,t" if causal else ""
    got, o, _ = _run(dev, orc, einsum, "attention", sp, [Q, K, V], params=params)
    o.close()
    f = orc.bf16_to_f64
    want_hm = orc.attention(f(_heads_first(Q)), f(_heads_first(K)), f(_heads_first(V)), 1.0 / np.sqrt(128.0), causal)
    want = np.moveaxis(want_hm.reshape(qshape[:1] + qshape[2:-1] + (qshape[1], 128)), -2, 1)
    assert rel_frobenius(got, orc.round_bf16(want)) <= BF16_TOL
    if einsum.startswith("bshd"):
        hm = {"b": sp["b"], "h": sp["h"], "s": sp["s"], "t": sp["t"], "d": sp["d"]}
        ref, o, _ = _run(dev, orc, "bhsd,bhtd,bhtd->bhsd", "attention", hm,
                         [np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (Q, K, V)], params=params)
        o.close()
        assert np.array_equal(got, ref.transpose(0, 2, 1, 3))


# ------------------------------------------------------------------ grouped-query attention

GQA_CASES = [
    # (B, G, R, S, T, splits of g, r, s, t, causal): Q [B, G, R, S, 128], K and V [B, G, T, 128]
    ((1, 2, 4, 384, 384), {"g": [0, 1, 2], "r": [0, 4], "s": _eq(384, 3), "t": _eq(384, 3)}, True),
    ((2, 3, 2, 200, 200), {"g": [0, 2, 3], "r": [0, 1, 2], "s": [0, 72, 200], "t": [0, 130, 200]}, True),
    ((1, 2, 3, 256, 384), {"g": [0, 2], "r": [0, 3], "s": [0, 128, 256], "t": [0, 64, 384]}, False),
]


@pytest.mark.parametrize("shape,sp,causal", GQA_CASES)
def test_gqa_attention_small(dev, orc, shape, sp, causal):
    """Query head g R + r reads key-value head g; splitting g splits the
    query heads with it (the pages' section 3.3)."""
    Bn, G, R, S, T = shape
    sp = dict(sp, b=_eq(Bn, Bn), d=[0, 128])
    Q = synth.normal_bf16(11, 0, (Bn, G, R, S, 128))
    K = synth.normal_bf16(11, 1, (Bn, G, T, 128))
    V = synth.normal_bf16(11, 2, (Bn, G, T, 128))
    got, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V],
                     params="causal=s,t" if causal else "")
    o.close()
    want = orc.attention(orc.bf16_to_f64(Q).reshape(Bn, G * R, S, 128), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                         1.0 / np.sqrt(128.0), causal)
    assert rel_frobenius(got, orc.round_bf16(want).reshape(Bn, G, R, S, 128)) <= BF16_TOL


def test_gqa_attention_8k_sampled_rows(dev, orc):
    """The pages' grouped-query shape: 32 query heads over 8 key-value heads,
    one 8,192-token sequence, 128-blocks on s and t, causal: 8 x 2,080
    tuples, 512 segments of 4 query heads each."""
    G, R, S = 8, 4, 8192
    sp = {"b": [0, 1], "g": _eq(G, G), "r": [0, R], "s": _eq(S, 64), "t": _eq(S, 64), "d": [0, 128]}
    Q = synth.normal_bf16(12, 0, (1, G, R, S, 128))
    K = synth.normal_bf16(12, 1, (1, G, S, 128))
    V = synth.normal_bf16(12, 2, (1, G, S, 128))
    got, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V], params="causal=s,t")
    rec, seg = o.tuples()
    o.close()
    assert rec.shape[0] == 8 * 2080 and len(seg) - 1 == 512
    rng = np.random.default_rng(4)
    ss = sorted(set([0, 1, 127, 128, 4095, 8191] + list(rng.integers(0, S, 6))))
    rows = np.array([(0, h, s) for h in (0, 3, 4, 17, 31) for s in ss])
    want = orc.attention_rows(orc.bf16_to_f64(Q).reshape(1, G * R, S, 128), orc.bf16_to_f64(K),
                              orc.bf16_to_f64(V), rows, 1.0 / np.sqrt(128.0), True)
    g = got.reshape(1, G * R, S, 128)[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert rel_frobenius(g, orc.round_bf16(want)) <= BF16_TOL
    assert np.isfinite(got).all()


def test_gqa_attention_128k_single_sequence(dev, orc):
    """The pages' longest workload: one 131,072-token sequence, 32 query heads
    over 8 key-value heads, 128-blocks on s and t, causal: 8 x 524,800 tuples
    (4.2 M) in 8,192 segments.  Inputs are drawn on the device (seeded N(0, 1)
    bf16, directly in the relation layout) and copied to the host for the
    oracle, which computes sampled rows against all of their keys."""
    import torch

    G, R, S = 8, 4, 131072
    n = S // 128
    sp = {"b": [0, 1], "g": _eq(G, G), "r": [0, R], "s": _eq(S, n), "t": _eq(S, n), "d": [0, 128]}
    op = dev.Op("bgrsd,bgtd,bgtd->bgrsd", "attention", sp, "causal=s,t")
    try:
        gen = torch.Generator(device="cuda").manual_seed(13)
        ins = [dev.alloc(r).normal_(generator=gen) for r in op.in_rels]
        out = dev.alloc(op.out_rel)
        op.run(ins, out)
        torch.cuda.synchronize()
        rec, seg = op.tuples()
        assert rec.shape[0] == G * n * (n + 1) // 2 and len(seg) - 1 == G * n
        host = [orc.Relation(r.shape, r.splits).unpack(bf16_bits(t)) for r, t in zip(op.in_rels, ins)]
        got = orc.bf16_to_f64(orc.Relation(op.out_rel.shape, op.out_rel.splits).unpack(bf16_bits(out)))
    finally:
        op.close()
    rng = np.random.default_rng(5)
    ss = sorted(set([0, 127, 128, 65535, 65536, S - 1] + list(rng.integers(0, S, 4))))
    rows = np.array([(0, h, s) for h in (0, 5, 18, 31) for s in ss])
    Q = orc.bf16_to_f64(host[0]).reshape(1, G * R, S, 128)
    want = orc.attention_rows(Q, orc.bf16_to_f64(host[1]), orc.bf16_to_f64(host[2]), rows, 1.0 / np.sqrt(128.0), True)
    g = got.reshape(1, G * R, S, 128)[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert rel_frobenius(g, orc.round_bf16(want)) <= BF16_TOL
    assert np.isfinite(got[0, :, :, ::4096]).all()


# ------------------------------------------------------------------ packed sequences

PACKED_CASES = [
    # (heads q, heads kv, S, sequence ends, s and t cuts, causal)
    (2, 2, 4096, [1024, 2560, 4096], [0, 1024, 2560, 4096], True),   # the pages' section 3.3 example
    (2, 2, 3000, [700, 1900, 3000], [0, 700, 3000], True),          # a block of two sequences; ends mid-tile
    (1, 1, 3000, [700, 1900, 3000], [0, 3000], False),              # one block of three, bidirectional
    (4, 2, 2000, [300, 301, 1250, 2000], [0, 301, 2000], True),     # grouped-query; a one-token sequence
]


@pytest.mark.parametrize("H,HK,S,ends,cuts,causal", PACKED_CASES)
def test_packed_attention(dev, orc, H, HK, S, ends, cuts, causal):
    """Sequences packed end to end along s and t (the pages' section 3.3):
    no query sees a key of another sequence, whichever sequence ends the
    decomposition cuts at."""
    R = H // HK
    sp = {"b": [0, 1], "g": _eq(HK, HK), "r": [0, R], "s": cuts, "t": cuts, "d": [0, 128]}
    Q = synth.normal_bf16(15, 0, (1, HK, R, S, 128))
    K = synth.normal_bf16(15, 1, (1, HK, S, 128))
    V = synth.normal_bf16(15, 2, (1, HK, S, 128))
    params = "packed=" + ",".join(map(str, ends)) + (";causal=s,t" if causal else "")
    got, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V], params=params)
    o.close()
    want = orc.attention(orc.bf16_to_f64(Q).reshape(1, H, S, 128), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                         1.0 / np.sqrt(128.0), causal, seq_ends=ends)
    assert rel_frobenius(got.reshape(1, H, S, 128), orc.round_bf16(want)) <= BF16_TOL
    assert np.isfinite(got).all()


@pytest.mark.parametrize("H,HK,S,ends,cuts,causal", [PACKED_CASES[0], PACKED_CASES[3]])
def test_packed_attention_token_major(dev, orc, H, HK, S, ends, cuts, causal):
    """Packed sequences on token-major relations (the heads inside a row): bit
    for bit the head-major result on the same values."""
    R = H // HK
    sp = {"b": [0, 1], "g": [0, HK], "r": [0, R], "s": cuts, "t": cuts, "d": [0, 128]}
    Q = synth.normal_bf16(25, 0, (1, HK, R, S, 128))
    K = synth.normal_bf16(25, 1, (1, HK, S, 128))
    V = synth.normal_bf16(25, 2, (1, HK, S, 128))
    params = "packed=" + ",".join(map(str, ends)) + (";causal=s,t" if causal else "")
    hm, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V], params=params)
    o.close()
    tm, o, _ = _run(dev, orc, "bsgrd,btgd,btgd->bsgrd", "attention", sp,
                    [np.ascontiguousarray(Q.transpose(0, 3, 1, 2, 4))] +
                    [np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (K, V)], params=params)
    o.close()
    assert np.array_equal(tm, hm.transpose(0, 3, 1, 2, 4))
    want = orc.attention(orc.bf16_to_f64(Q).reshape(1, H, S, 128), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                         1.0 / np.sqrt(128.0), causal, seq_ends=ends)
    assert rel_frobenius(hm.reshape(1, H, S, 128), orc.round_bf16(want)) <= BF16_TOL


# ------------------------------------------------------------------ fp16 relations

F16_CONTRACT_CASES = [
    ("ij,jk->ik", {"i": [0, 77, 200], "j": [0, 96, 320], "k": [0, 64, 136]}),
    ("ij,kj->ik", {"i": [0, 300], "j": [0, 128, 256], "k": [0, 264]}),
    ("ji,jk->ik", {"i": [0, 136], "j": [0, 64, 128], "k": [0, 40, 96]}),
    ("bd,df->bf", {"b": [0, 256, 512], "d": [0, 512, 1024], "f": [0, 384, 776]}),
]


@pytest.mark.parametrize("einsum,sp", F16_CONTRACT_CASES)
def test_contract_f16(dev, orc, einsum, sp):
    """IEEE half relations (the pages' blocks run in fp16): fp16 in, fp32
    accumulate, fp16 or fp32 out, fused and unfused (partials, then SUM)."""
    import torch

    from tensor_relational_join_amd.binding import JA_F16, JA_F32

    lhs, out = einsum.split("->")
    shapes = [tuple(sp[c][-1] for c in s) for s in lhs.split(",")]
    X = synth.normal_f16(21, 0, shapes[0])
    W = synth.normal_f16(21, 1, shapes[1], std=0.02)
    exact = orc.einsum(einsum, orc.f16_to_f64(X), orc.f16_to_f64(W))
    got, o, ins = _run(dev, orc, einsum, "contract", sp, [X, W], in_dtypes=[JA_F16, JA_F16], out_dtype=JA_F16)
    try:
        want = orc.round_f16(exact)
        assert rel_frobenius(got, want) <= BF16_TOL
        assert np.mean(got == want) > 0.9  # nearly every element is the correctly rounded fp32 sum
        part = o.partial_buffer()
        o.kernel(ins, part)
        out2 = dev.alloc(o.out_rel)
        o.agg(part, out2)
        torch.cuda.synchronize()
        orel = orc.Relation([sp[c][-1] for c in out], [sp[c] for c in out])
        assert rel_frobenius(orc.f16_to_f64(orel.unpack(bf16_bits(out2))), want) <= BF16_TOL
    finally:
        o.close()
    got32, o, _ = _run(dev, orc, einsum, "contract", sp, [X, W], in_dtypes=[JA_F16, JA_F16], out_dtype=JA_F32)
    o.close()
    assert rel_inf(got32, exact) <= 1e-5  # fp32 accumulation of exact fp16 products


@pytest.mark.parametrize("causal,packed", [(True, None), (False, None), (True, [200, 512])])
def test_attention_f16(dev, orc, causal, packed):
    """fp16 Q, K, V, O: the scores multiply in fp16 and V needs no conversion."""
    from tensor_relational_join_amd.binding import JA_F16

    G, R, S = 2, 2, 512
    cuts = [0, 200, 512] if packed else _eq(S, 4)
    sp = {"b": [0, 1], "g": _eq(G, G), "r": [0, R], "s": cuts, "t": cuts, "d": [0, 128]}
    Q = synth.normal_f16(22, 0, (1, G, R, S, 128))
    K = synth.normal_f16(22, 1, (1, G, S, 128))
    V = synth.normal_f16(22, 2, (1, G, S, 128))
    params = ";".join(p for p in ("causal=s,t" if causal else "",
                                  "packed=" + ",".join(map(str, packed)) if packed else "") if p)
    got, o, _ = _run(dev, orc, "bgrsd,bgtd,bgtd->bgrsd", "attention", sp, [Q, K, V], params=params,
                     in_dtypes=[JA_F16] * 3, out_dtype=JA_F16)
    o.close()
    want = orc.attention(orc.f16_to_f64(Q).reshape(1, G * R, S, 128), orc.f16_to_f64(K), orc.f16_to_f64(V),
                         1.0 / np.sqrt(128.0), causal, seq_ends=packed)
    assert rel_frobenius(got.reshape(1, G * R, S, 128), orc.round_f16(want)) <= BF16_TOL


@pytest.mark.parametrize("op", ["rmsnorm", "swiglu", "add"])
def test_norm_and_elementwise_f16(dev, orc, op):
    from tensor_relational_join_amd.binding import JA_F16

    if op == "rmsnorm":
        R, D = 300, 4096
        x = synth.normal_f16(23, 0, (R, D))
        gn = synth.normal_f16(23, 1, (D,), mean=1.0, std=0.1)
        got, o, _ = _run(dev, orc, "rd,d->rd", "rmsnorm", {"r": [0, 100, 300], "d": _eq(D, 8)}, [x, gn],
                         params="eps=1e-6", in_dtypes=[JA_F16] * 2, out_dtype=JA_F16)
        want = orc.round_f16(orc.rmsnorm(orc.f16_to_f64(x), orc.f16_to_f64(gn), 1e-6))
    else:
        R, F = 64, 1000
        a = synth.normal_f16(24, 0, (R, F))
        b = synth.normal_f16(24, 1, (R, F))
        got, o, _ = _run(dev, orc, "rf,rf->rf", op, {"r": [0, R], "f": [0, 504, 1000]}, [a, b],
                         in_dtypes=[JA_F16] * 2, out_dtype=JA_F16)
        af, bf = orc.f16_to_f64(a), orc.f16_to_f64(b)
        want = orc.round_f16(orc.swiglu(af, bf) if op == "swiglu" else orc.add(af, bf))
    o.close()
    assert rel_frobenius(got, want) <= BF16_TOL
    assert np.mean(got == want) > 0.99


# ------------------------------------------------------------------ RMSNorm, SwiGLU, add

@pytest.mark.parametrize("R,D,rsp,dsp", [
    (64, 512, [0, 64], _eq(512, 4)),
    (70, 200, [0, 5, 70], [0, 7, 100, 200]),      # unaligned widths: element path
    (8192, 4096, [0, 8192], _eq(4096, 8)),         # x [8192, 4096], d split into 8 blocks
    # rows held in registers: several row blocks, 6 and 2 vectors per lane
    (300, 2048, [0, 100, 300], _eq(2048, 2)),
    (10, 3072, [0, 3, 10], _eq(3072, 3)),
    (5, 1024, [0, 5], [0, 1024]),
    # more rows than resident wavefronts, so each walks several rows and
    # prefetches the next, across row blocks; 16 vectors per lane
    (5000, 1024, [0, 1999, 5000], _eq(1024, 2)),
    (2500, 8192, [0, 1300, 2500], [0, 8192]),
])
def test_rmsnorm(dev, orc, R, D, rsp, dsp):
    x = synth.normal_bf16(4, 0, (R, D))
    g = synth.normal_bf16(4, 1, (D,), mean=1.0, std=0.1)
    sp = {"r": rsp, "d": dsp}
    got, o, _ = _run(dev, orc, "rd,d->rd", "rmsnorm", sp, [x, g], params="eps=1e-6")
    o.close()
    want = orc.round_bf16(orc.rmsnorm(orc.bf16_to_f64(x), orc.bf16_to_f64(g), 1e-6))
    assert rel_frobenius(got, want) <= BF16_TOL
    assert np.mean(got == want) > 0.99


@pytest.mark.parametrize("op,R,F,fsp", [
    ("swiglu", 33, 100, [0, 37, 100]),
    ("swiglu", 8192, 11008, _eq(11008, 8)),        # g, u [8192, 11008], 1:1 join over 8 blocks
    ("add", 64, 4096, _eq(4096, 8)),
    ("add", 3, 7, [0, 7]),                         # tail shorter than one vector
])
def test_elementwise(dev, orc, op, R, F, fsp):
    a = synth.normal_bf16(6, 0, (R, F))
    b = synth.normal_bf16(6, 1, (R, F))
    sp = {"r": [0, R], "f": fsp}
    got, o, _ = _run(dev, orc, "rf,rf->rf", op, sp, [a, b])
    o.close()
    af, bf = orc.bf16_to_f64(a), orc.bf16_to_f64(b)
    want = orc.round_bf16(orc.swiglu(af, bf) if op == "swiglu" else orc.add(af, bf))
    assert rel_frobenius(got, want) <= BF16_TOL
    assert np.mean(got == want) > 0.99


# ------------------------------------------------------------------ repartition (bit-exact)

def _repart_case(dev, orc, shape_src, src_splits, shape_dst, dst_splits, vshape=None, perm=None, dtype="bf16",
                 seed=0):
    import torch

    from tensor_relational_join_amd import binding as B

    jd = B.JA_BF16 if dtype == "bf16" else B.JA_F32
    s_rel = B.Relation(shape_src, splits=src_splits, dtype=jd)
    d_rel = B.Relation(shape_dst, splits=dst_splits, dtype=jd)
    view = B.make_view(vshape, perm) if vshape is not None else None
    rp = dev.Repart(s_rel, d_rel, view)
    try:
        rng = np.random.default_rng(seed)
        if dtype == "bf16":
            dense = rng.integers(0, 65536, size=shape_src, dtype=np.uint32).astype(np.uint16)
        else:
            dense = rng.integers(0, 2 ** 32, size=shape_src, dtype=np.uint64).astype(np.uint32)
        os_rel = orc.Relation(shape_src, src_splits)
        od_rel = orc.Relation(shape_dst, dst_splits)
        flat = os_rel.pack(dense)
        src_t = torch.from_numpy(flat.view(np.int16 if dtype == "bf16" else np.int32)).cuda()
        dst_t = torch.zeros(od_rel.shape and int(np.prod(shape_dst)), dtype=src_t.dtype, device="cuda")
        rp.run(src_t, dst_t)
        torch.cuda.synchronize()
        got = dst_t.cpu().numpy().view(np.uint16 if dtype == "bf16" else np.uint32)
        want = orc.repartition(os_rel, flat, od_rel, vshape, perm)
        assert np.array_equal(got, want)
        return rp.n_atoms, rp.n_tasks
    finally:
        rp.close()


def test_repartition_section_5_3_example(dev, orc):
    n_atoms, _ = _repart_case(dev, orc, (256, 256), [[0, 128, 256], [0, 256]], (256, 256),
                              [[0, 64, 128, 192, 256], [0, 256]])
    assert n_atoms == 4


@pytest.mark.parametrize("seed", range(6))
def test_repartition_random_blockings(dev, orc, seed):
    rng = np.random.default_rng(100 + seed)
    rank = int(rng.integers(1, 4))
    shape = tuple(int(x) for x in rng.integers(1, 40, rank))

    def rand_splits(n):
        k = int(rng.integers(0, min(4, n)))
        return [0] + sorted(set(int(x) for x in rng.integers(1, n, k))) + [n] if n > 1 else [0, n]

    src = [rand_splits(n) for n in shape]
    dst = [rand_splits(n) for n in shape]
    _repart_case(dev, orc, shape, src, shape, dst, dtype="bf16" if seed % 2 else "f32", seed=seed)


def test_repartition_views(dev, orc):
    # transpose of a blocked matrix
    _repart_case(dev, orc, (24, 40), [[0, 10, 24], [0, 16, 40]], (40, 24), [[0, 8, 40], [0, 24]],
                 vshape=(24, 40), perm=(1, 0), seed=3)
    # split a dim and permute (rank 2 -> rank 3)
    _repart_case(dev, orc, (12, 16), [[0, 5, 12], [0, 16]], (4, 12, 4), [[0, 2, 4], [0, 12], [0, 3, 4]],
                 vshape=(12, 4, 4), perm=(1, 0, 2), seed=4)


def test_repartition_llama_views_full_size(dev, orc):
    """Token-major QKV [8192, 12288] blocked 2x2 -> head-major [3, 4, 32, 2048, 128]
    with [1,1,1,128,128] blocks, and attention output heads -> tokens."""
    na, nt = _repart_case(dev, orc, (8192, 12288), [_eq(8192, 2), _eq(12288, 2)], (3, 4, 32, 2048, 128),
                          [_eq(3, 3), _eq(4, 4), _eq(32, 32), _eq(2048, 16), [0, 128]],
                          vshape=(4, 2048, 3, 32, 128), perm=(2, 0, 3, 1, 4), seed=5)
    assert na == 6144
    _repart_case(dev, orc, (4, 32, 2048, 128), [_eq(4, 4), _eq(32, 32), _eq(2048, 16), [0, 128]], (8192, 4096),
                 [_eq(8192, 2), _eq(4096, 2)], vshape=(4, 32, 2048, 128), perm=(0, 2, 1, 3), seed=6)
    _repart_case(dev, orc, (8192, 4096), [_eq(8192, 2), _eq(4096, 8)], (8192, 4096),
                 [_eq(8192, 2), _eq(4096, 2)], seed=7)


def test_repartition_unit_dimensions(dev, orc):
    _repart_case(dev, orc, (256, 768), [_eq(256, 2), _eq(768, 2)], (3, 1, 2, 256, 128),
                 [_eq(3, 3), [0, 1], _eq(2, 2), _eq(256, 2), [0, 128]], vshape=(1, 256, 3, 2, 128),
                 perm=(2, 0, 3, 1, 4), seed=8)
    _repart_case(dev, orc, (1, 1), [[0, 1], [0, 1]], (1,), [[0, 1]], vshape=(1,), perm=(0,), dtype="f32", seed=9)


# ------------------------------------------------------------------ one-shot entry points

def _one_shot(dev, orc, einsum, op, splits, dense_inputs, params="", in_dtypes=None, out_dtype=None):
    """Run an operator through ja_einsum (plan, upload and run in one call, with
    a caller-owned workspace of the queried size) and unpack its output."""
    import torch

    from tensor_relational_join_amd import binding as B

    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    in_dtypes = in_dtypes or [B.JA_BF16] * len(ins)
    out_dtype = B.JA_BF16 if out_dtype is None else out_dtype
    spec = B.ja_spec_create(einsum, op, params)
    decomp = None
    try:
        letters = B.ja_spec_letters(spec)
        decomp = B.ja_decomp_create(spec, [splits[c][-1] for c in letters], [len(splits[c]) - 1 for c in letters],
                                    [list(splits[c]) for c in letters])
        in_rels = [dev.relation_for(s, splits, dt) for s, dt in zip(ins, in_dtypes)]
        out_rel = dev.relation_for(out, splits, out_dtype)
        dev_ins = []
        for s, x, dt in zip(ins, dense_inputs, in_dtypes):
            flat = orc.Relation([splits[c][-1] for c in s], [splits[c] for c in s]).pack(x)
            dev_ins.append(to_dev_bf16(flat) if dt == B.JA_BF16 else to_dev_f32(flat))
        out_t = dev.alloc(out_rel)
        need = B.ja_einsum_workspace_bytes(spec, decomp, in_rels, out_rel)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        B.ja_einsum(spec, decomp, in_rels, [t.data_ptr() for t in dev_ins], out_rel, out_t.data_ptr(),
                    ws.data_ptr(), need)
        torch.cuda.synchronize()
        orel = orc.Relation([splits[c][-1] for c in out], [splits[c] for c in out])
        host = bf16_bits(out_t) if out_dtype == B.JA_BF16 else f32_host(out_t)
        res = orel.unpack(host)
        if out_dtype == B.JA_BF16:
            res = orc.bf16_to_f64(res)
        return res.astype(np.float64), dev_ins
    finally:
        if decomp is not None:
            B.ja_decomp_destroy(decomp)
        B.ja_spec_destroy(spec)


def test_one_shot_einsum_fp32(dev, orc):
    from tensor_relational_join_amd.binding import JA_F32

    A = synth.uniform(21, 0, (64, 64))
    Bm = synth.uniform(21, 1, (64, 64))
    sp = {c: _eq(64, 2) for c in "ijk"}
    got, _ = _one_shot(dev, orc, "ij,jk->ik", "contract", sp, [A, Bm], in_dtypes=[JA_F32, JA_F32],
                       out_dtype=JA_F32)
    assert rel_inf(got, orc.einsum("ij,jk->ik", A, Bm)) <= FP32_TOL


def test_one_shot_einsum_bf16_matches_plan_path(dev, orc):
    """The one-shot call and the plan API run the same kernels on the same
    tuple list, so their outputs agree bit for bit; both meet the oracle bar."""
    sp = {"i": [0, 144, 300], "j": [0, 104, 520], "k": [0, 128, 256, 328]}
    X = synth.normal_bf16(22, 0, (300, 520))
    W = synth.normal_bf16(22, 1, (520, 328), std=0.02)
    got, _ = _one_shot(dev, orc, "ij,jk->ik", "contract", sp, [X, W])
    want = orc.round_bf16(orc.einsum("ij,jk->ik", orc.bf16_to_f64(X), orc.bf16_to_f64(W)))
    assert rel_frobenius(got, want) <= BF16_TOL
    got2, o, _ = _run(dev, orc, "ij,jk->ik", "contract", sp, [X, W])
    o.close()
    assert np.array_equal(got, got2)


def test_one_shot_attention(dev, orc):
    Bn, H, S = 1, 2, 384
    sp = {"b": [0, 1], "h": _eq(H, H), "s": _eq(S, 3), "t": _eq(S, 2), "d": [0, 128]}
    Q = synth.normal_bf16(23, 0, (Bn, H, S, 128))
    K = synth.normal_bf16(23, 1, (Bn, H, S, 128))
    V = synth.normal_bf16(23, 2, (Bn, H, S, 128))
    got, _ = _one_shot(dev, orc, "bhsd,bhtd,bhtd->bhsd", "attention", sp, [Q, K, V], params="causal=s,t")
    want = orc.round_bf16(orc.attention(orc.bf16_to_f64(Q), orc.bf16_to_f64(K), orc.bf16_to_f64(V),
                                        1.0 / np.sqrt(128.0), True))
    assert rel_frobenius(got, want) <= BF16_TOL


def test_one_shot_repartition(dev, orc):
    """ja_repartition (tables built, uploaded and run in one call) gives the
    same bytes as the oracle's repartition, with and without a view."""
    import torch

    from tensor_relational_join_amd import binding as B

    cases = [((256, 256), [[0, 128, 256], [0, 256]], (256, 256), [[0, 64, 128, 192, 256], [0, 256]], None, None),
             ((24, 40), [[0, 10, 24], [0, 16, 40]], (40, 24), [[0, 8, 40], [0, 24]], (24, 40), (1, 0))]
    for n, (ss, ssp, ds, dsp, vshape, perm) in enumerate(cases):
        s_rel = B.Relation(ss, splits=ssp, dtype=B.JA_BF16)
        d_rel = B.Relation(ds, splits=dsp, dtype=B.JA_BF16)
        view = B.make_view(vshape, perm) if vshape is not None else None
        dense = np.random.default_rng(40 + n).integers(0, 65536, size=ss, dtype=np.uint32).astype(np.uint16)
        os_rel, od_rel = orc.Relation(ss, ssp), orc.Relation(ds, dsp)
        flat = os_rel.pack(dense)
        src_t = torch.from_numpy(flat.view(np.int16)).cuda()
        dst_t = torch.zeros(int(np.prod(ds)), dtype=torch.int16, device="cuda")
        need = B.ja_repartition_workspace_bytes(s_rel, d_rel, view)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        B.ja_repartition(s_rel, src_t.data_ptr(), d_rel, dst_t.data_ptr(), view, ws.data_ptr(), need)
        torch.cuda.synchronize()
        got = dst_t.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, orc.repartition(os_rel, flat, od_rel, vshape, perm))
