"""Attention as the three phases of Definition 3.7 with the per-tuple results
materialised ("Every Kernel Is a Join", paperpeel full text, section 3.2):
ja_kernel writes every kept tuple's softmax triple (m, l, acc) per query row,
ja_agg with JA_AGG_SOFTMAX folds each segment's triples (the aggregation need
not be addition, section 5.2) and writes O.

Partials against the oracle's per-tuple triples: a triple is defined only up
to its reference maximum, so the unique parts are compared -- the
log-sum-exp m + ln l (absolute 2e-3) and the normalised values acc / l
(relative Frobenius 2e-3); rows that see no key of their tuple must hold the
identity (-inf, 0, 0) exactly.  The aggregated O against two-pass attention
at the bf16 bar, and against the fused kernel's O."""
import itertools

import numpy as np
import pytest

from gpu_helpers import bf16_bits, f32_host, record, rel_frobenius, to_dev_bf16, to_dev_f16
from tensor_relational_join_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
PROW = 132


def _eq(n, q):
    base, extra = divmod(n, q)
    p = [0]
    for i in range(q):
        p.append(p[-1] + base + (i < extra))
    return p


CASES = [
    # (einsum, Q shape, KV shape, splits, params, dtype)
    ("bhsd,bhtd,bhtd->bhsd", (1, 2, 300, 128), (1, 2, 300, 128),
     {"b": [0, 1], "h": [0, 1, 2], "s": [0, 100, 300], "t": [0, 50, 180, 300]}, "causal=s,t", "bf16"),
    ("bhsd,bhtd,bhtd->bhsd", (2, 2, 256, 128), (2, 2, 384, 128),
     {"b": [0, 1, 2], "h": [0, 2], "s": [0, 128, 256], "t": [0, 64, 384]}, "", "bf16"),
    ("bhsd,bhtd,bhtd->bhsd", (1, 2, 384, 128), (1, 2, 384, 128),
     {"b": [0, 1], "h": [0, 1, 2], "s": _eq(384, 3), "t": _eq(384, 3)}, "causal=s,t", "f16"),
    # grouped-query: 2 query heads per key-value head
    ("bgrsd,bgtd,bgtd->bgrsd", (1, 2, 2, 256, 128), (1, 2, 256, 128),
     {"b": [0, 1], "g": [0, 1, 2], "r": [0, 2], "s": [0, 128, 256], "t": [0, 128, 256]}, "causal=s,t", "bf16"),
    # packed sequences ending at 100, 260, 400
    ("bhsd,bhtd,bhtd->bhsd", (1, 1, 400, 128), (1, 1, 400, 128),
     {"b": [0, 1], "h": [0, 1], "s": [0, 100, 260, 400], "t": [0, 100, 260, 400]}, "causal=s,t;packed=100,260,400",
     "bf16"),
]


def _flat_heads(x, einsum):
    """[b, (g, r) or h, s, d] with the query heads flattened."""
    return x.reshape(x.shape[0], -1, x.shape[-2], x.shape[-1]) if einsum.startswith("bgr") else x


@pytest.mark.parametrize("case", range(len(CASES)))
def test_unfused_attention_partials_and_softmax_aggregation(orc, case):
    import torch

    from tensor_relational_join_amd import device as dev
    from tensor_relational_join_amd.binding import JA_AGG_SOFTMAX, JA_AGG_SUM, JA_BF16, JA_F16, JaError

    einsum, qshape, kvshape, sp, params, dt = CASES[case]
    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    sp = dict(sp, d=[0, 128])
    jdt = JA_BF16 if dt == "bf16" else JA_F16
    gen = synth.normal_bf16 if dt == "bf16" else synth.normal_f16
    dec = orc.bf16_to_f64 if dt == "bf16" else orc.f16_to_f64
    rnd = orc.round_bf16 if dt == "bf16" else orc.round_f16
    put = to_dev_bf16 if dt == "bf16" else to_dev_f16
    Q, K, V = gen(30 + case, 0, qshape), gen(30 + case, 1, kvshape), gen(30 + case, 2, kvshape)
    o = dev.Op(einsum, "attention", sp, params, [jdt] * 3, jdt)
    try:
        dins = [put(orc.Relation([sp[c][-1] for c in x], [sp[c] for c in x]).pack(a)) for x, a in zip(ins, (Q, K, V))]
        part = o.partial_buffer()
        o.kernel(dins, part)
        out_t = dev.alloc(o.out_rel)
        o.agg(part, out_t, op=JA_AGG_SOFTMAX)
        fused = dev.alloc(o.out_rel)
        o.run(dins, fused)
        torch.cuda.synchronize()
        with pytest.raises(JaError):  # attention partials take the softmax aggregation only
            o.agg(part, out_t, op=JA_AGG_SUM)
        rec, seg = o.tuples()
        letters = o.letters
        p = f32_host(part)
        orel = orc.Relation([sp[c][-1] for c in out], [sp[c] for c in out])
        got = dec(orel.unpack(bf16_bits(out_t)))
        got_fused = dec(orel.unpack(bf16_bits(fused)))
    finally:
        o.close()
    causal = "causal" in params
    ends = [int(x) for x in params.split("packed=")[1].split(",")] if "packed=" in params else None
    qf, kf, vf = (dec(a) for a in (Q, K, V))
    S = qshape[-2]
    want = rnd(orc.attention(_flat_heads(qf, einsum), kf, vf, 1.0 / np.sqrt(128.0), causal, ends)).reshape(got.shape)
    err = rel_frobenius(got, want)
    assert err <= TOL
    assert rel_frobenius(got_fused, want) <= TOL
    # per-tuple partials against the oracle's triples, tuple by tuple in tuple order
    bsp = [sp[c] for c in ins[0][:-2]]  # the query batch letters (b, or b g r)
    tri = orc.attention_triples(_flat_heads(qf, einsum), kf, vf, sp["s"], sp["t"], 1.0 / np.sqrt(128.0), causal, ends)
    tri = {k: (m, l, a) for k, m, l, a in tri}
    off = 0
    lse_err, nv, na, nid = 0.0, [], [], 0
    for r in rec.tolist():
        iv = [r[letters.index(c)] for c in ins[0][:-2]]
        si, ti = r[letters.index("s")], r[letters.index("t")]
        s0, s1 = sp["s"][si], sp["s"][si + 1]
        ranges = [range(b[i], b[i + 1]) for b, i in zip(bsp, iv)]
        bhs = list(itertools.product(*ranges))
        blk = p[off:off + len(bhs) * (s1 - s0) * PROW].reshape(len(bhs), s1 - s0, PROW)
        off += blk.size
        for j, idx in enumerate(bhs):
            b = idx[0]
            h = int(np.ravel_multi_index(idx[1:], qshape[1:-2])) if len(idx) > 1 else 0
            m, l, acc = tri[(b, h, si, ti)]
            gm, gl, gacc = blk[j, :, 0].astype(np.float64), blk[j, :, 1].astype(np.float64), blk[j, :, 4:]
            empty = ~np.isfinite(m)
            nid += int(empty.sum())
            assert np.all(gm[empty] == -np.inf) and np.all(gl[empty] == 0) and not gacc[empty].any()
            ok = ~empty
            d = np.abs(gm[ok] + np.log(gl[ok]) - (m[ok] + np.log(l[ok])))
            lse_err = max(lse_err, float(d.max(initial=0.0)))
            nv.append(gacc[ok] / gl[ok][:, None])
            na.append(acc[ok] / l[ok][:, None])
    assert off <= part.numel()
    norm_err = rel_frobenius(np.concatenate(nv), np.concatenate(na))
    record("unfused_attention", case=case, out_rel_frobenius=err, lse_abs=lse_err, partial_rel_frobenius=norm_err,
           identity_rows=nid)
    assert lse_err <= 2e-3
    assert norm_err <= TOL
    if causal and case == 0:
        assert nid > 0  # the uneven blocks leave rows that see no key of some tuple
