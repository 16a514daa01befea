"""The LLaMA-shaped block as a graph of join-agg operators on the GPU,
against the oracle.

Per-step parity (the bar): every step's GPU output is compared with the
oracle applied to that step's GPU inputs -- full tensors for the
memory-bound steps and at reduced shapes, sampled outputs for the full-size
contractions and attention, bit-exact for the two repartitions -- at the
bf16 tolerance (relative Frobenius <= 2e-3).

End-to-end chain: the block output is also compared with the oracle's own
chain from the block inputs.  At the reduced shapes it is held to the same
2e-3, and so are the all-half blocks at full size.  The full-size bf16
blocks are held to CHAIN_TOL_FULL = 5e-3: attention rounds P
to IEEE half for its P V product, which keeps attention itself within 2e-3
but changes O enough to flip downstream bf16 roundings, and the FFN carries
those to y.  The oracle alone shows it (tests/test_chain_tolerance.py): with
only P rounded to half, its full-size chain moves by 3.4-3.8e-3; with P kept
in float32, by nothing.  The measured errors are recorded through
JA_PARITY_RECORD.  The full-size tokens span each sequence, so queries that
read every off-diagonal key block feed the comparison.

Every test runs both forms of the block: the residual adds and SwiGLU as
launches of their own, and fused into the contractions that produce their
inputs (checked per step as contraction + residual and gate-and-up +
SwiGLU, against the oracle's fused rounding points)."""
import itertools

import numpy as np
import pytest

from gpu_helpers import bf16_bits, record, rel_frobenius, to_dev_bf16, to_dev_f16
from tensor_relational_join_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
CHAIN_TOL = 2e-3
CHAIN_TOL_FULL = 5e-3  # derived in tests/test_chain_tolerance.py


def _fmt(orc, dt):
    """(decode, round, upload) of the block's 16-bit format: "bf16" or "f16"."""
    if dt == "f16":
        return orc.f16_to_f64, orc.round_f16, to_dev_f16
    return orc.bf16_to_f64, orc.round_bf16, to_dev_bf16


def _run_block(orc, batch, seq, dm, heads, ffn, seed, kv_heads=None, fused=False, dt="bf16", layout="tokens",
               split_small=True):
    import torch

    from tensor_relational_join_amd.binding import JA_BF16, JA_F16
    from tensor_relational_join_amd.block import LlamaBlock
    from tensor_relational_join_amd.device import alloc

    put = _fmt(orc, dt)[2]
    pack = lambda rel, bits: put(orc.Relation(rel.shape, rel.splits).pack(bits))  # noqa: E731
    blk = LlamaBlock(batch, seq, dm, heads, ffn, kv_heads=kv_heads, fused=fused,
                     dtype=JA_F16 if dt == "f16" else JA_BF16, layout=layout, split_small=split_small)
    inp = synth.llama_block_inputs(seed, batch, seq, dm, ffn, qkv_cols=blk.qkv_cols, dtype=dt)
    x = pack(blk.x_rel, inp["x"])
    w = {k: pack(rel, inp[k]) for k, rel in blk.w_rel.items()}
    w["g1"] = pack(blk.g_rel, inp["g1"])
    w["g2"] = pack(blk.ops["norm2"].in_rels[1], inp["g2"])
    y = alloc(blk.y_rel)
    blk.forward(x, w, y)
    torch.cuda.synchronize()
    return blk, inp, x, y


def _check_steps(orc, blk, inp, y, sampled: bool, dt="bf16"):
    """Each step against the oracle on the GPU's inputs to that step.
    Returns {step: error}; repartitions report 0.0 when bit-exact."""
    o, b = blk.ops, blk.buf
    batch, seq, dm, heads, ffn, T = blk.batch, blk.seq, blk.dm, blk.heads, blk.ffn, blk.T
    f64, rnd, _ = _fmt(orc, dt)

    def _unpack(orc, rel, t):
        return f64(orc.Relation(rel.shape, rel.splits).unpack(bf16_bits(t)))

    rng = np.random.default_rng(2)
    errs = {}

    def contract(name, a_rel, a_buf, w_name, out_rel, out_buf, N, blockN, residual=None):
        """out = A W (w_name "w_gu": silu(A W_gate) * (A W_up); residual: + R),
        against the oracle on the GPU's A (and R)."""
        A = _unpack(orc, a_rel, a_buf)
        got = _unpack(orc, out_rel, out_buf)
        if sampled:
            rows = sorted(set([0, 1, T // 2 - 1, T // 2, T - 1] + list(rng.integers(0, T, 24))))
            cols = sorted(set([0, 1, 127, 128, blockN - 1, blockN, N - 1] + list(rng.integers(0, N, 24))))
            pts = np.array(list(itertools.product(rows, cols)))
            prod = lambda W: orc.einsum_points("ij,jk->ik", A, W, pts)
            if w_name == "w_gu":
                want = orc.swiglu(prod(f64(inp["w_gate"])), prod(f64(inp["w_up"])))
            else:
                want = prod(f64(inp[w_name]))
            if residual is not None:
                want = orc.add(want, residual[pts[:, 0], pts[:, 1]])
            errs[name] = rel_frobenius(got[pts[:, 0], pts[:, 1]], rnd(want))
        else:
            if w_name == "w_gu":
                want = orc.contract_swiglu("td,dfc->tf", A, f64(inp["w_gu"]))
            elif residual is not None:
                want = orc.contract_residual("ij,jk->ik", A, f64(inp[w_name]), residual)
            else:
                want = orc.matmul(A, f64(inp[w_name]))
            errs[name] = rel_frobenius(got, rnd(want))

    xd = f64(inp["x"])
    h1 = _unpack(orc, o["norm1"].out_rel, b["h1"])
    errs["norm1"] = rel_frobenius(h1, rnd(orc.rmsnorm(xd, f64(inp["g1"]), blk.eps)))
    N = blk.qkv_cols
    tok = blk.layout == "tokens"
    contract("qkv", o["norm1"].out_rel, b["h1"], "w_qkv", o["qkv"].out_rel, b["qkv"], N,
             dm if blk.gqa or tok else N // 2)
    qr = o["qkv"].out_rel
    kv, rep = blk.kv_heads, heads // blk.kv_heads
    if tok:
        # attention reads the projection's three contiguous token-major parts as they are
        flat = f64(bf16_bits(b["qkv"]))
        nq, nk = T * dm, T * kv * 128
        Qd = flat[:nq].reshape(batch, seq, heads, 128).transpose(0, 2, 1, 3)
        Kd = flat[nq:nq + nk].reshape(batch, seq, kv, 128).transpose(0, 2, 1, 3)
        Vd = flat[nq + nk:].reshape(batch, seq, kv, 128).transpose(0, 2, 1, 3)
    elif not blk.gqa:
        hr = blk.heads_rel
        want_heads = orc.repartition(orc.Relation(qr.shape, qr.splits), bf16_bits(b["qkv"]),
                                     orc.Relation(hr.shape, hr.splits), (batch, seq, 3, heads, 128), (2, 0, 3, 1, 4))
        heads_bits = bf16_bits(b["heads"])
        errs["to_heads"] = 0.0 if np.array_equal(heads_bits, want_heads) else 1.0
        Qd, Kd, Vd = f64(orc.Relation(hr.shape, hr.splits).unpack(heads_bits))
    else:
        # the projection's output is three contiguous [T, *] parts: Q heads, K heads, V heads
        flat = bf16_bits(b["qkv"])
        nq, nk = T * dm, T * kv * 128
        parts = {"q": flat[:nq], "k": flat[nq:nq + nk], "v": flat[nq + nk:]}
        views = {"q": ((batch, seq, kv, rep, 128), (0, 2, 3, 1, 4)), "k": ((batch, seq, kv, 128), (0, 2, 1, 3)),
                 "v": ((batch, seq, kv, 128), (0, 2, 1, 3))}
        ok, dense = True, {}
        for name, rel in zip("qkv", o["attn"].in_rels):
            pr = blk.part_rel[name]
            want_p = orc.repartition(orc.Relation(pr.shape, pr.splits), parts[name],
                                     orc.Relation(rel.shape, rel.splits), *views[name])
            got_p = bf16_bits(b[name])
            ok = ok and np.array_equal(got_p, want_p)
            dense[name] = f64(orc.Relation(rel.shape, rel.splits).unpack(got_p))
        errs["to_heads"] = 0.0 if ok else 1.0
        Qd, Kd, Vd = dense["q"].reshape(batch, heads, seq, 128), dense["k"], dense["v"]
    Od = _unpack(orc, o["attn"].out_rel, b["O"])
    Od = Od.reshape(batch, seq, heads, 128).transpose(0, 2, 1, 3) if tok else Od.reshape(batch, heads, seq, 128)
    if sampled:
        ss = [0, 1, 127, 128, 1000, seq - 1]
        rows = np.array([(bb, hh, s) for bb, hh in [(0, 0), (batch // 2, heads // 2), (batch - 1, heads - 1)]
                         for s in ss])
    else:
        rows = np.array(list(itertools.product(range(batch), range(heads), range(seq))))
    want = rnd(orc.attention_rows(Qd, Kd, Vd, rows, 1.0 / np.sqrt(128.0), True))
    errs["attn"] = rel_frobenius(Od[rows[:, 0], rows[:, 1], rows[:, 2]], want)
    oproj = o["oproj_add" if blk.fused else "oproj"]
    ar, orl = o["attn"].out_rel, oproj.in_rels[0]
    if not tok:
        view = ((batch, kv, rep, seq, 128), (0, 3, 1, 2, 4)) if blk.gqa else ((batch, heads, seq, 128), (0, 2, 1, 3))
        want_o = orc.repartition(orc.Relation(ar.shape, ar.splits), bf16_bits(b["O"]),
                                 orc.Relation(orl.shape, orl.splits), *view)
        errs["to_tokens"] = 0.0 if np.array_equal(bf16_bits(b["o"]), want_o) else 1.0
    else:
        assert b["o"].data_ptr() == b["O"].data_ptr()
    if blk.fused:
        contract("oproj_add", orl, b["o"], "w_o", oproj.out_rel, b["x2"], dm, dm // 2, residual=xd)
        x2 = _unpack(orc, oproj.out_rel, b["x2"])
    else:
        contract("oproj", orl, b["o"], "w_o", o["oproj"].out_rel, b["a"], dm, dm // 2)
        x2 = _unpack(orc, o["add1"].out_rel, b["x2"])
        errs["add1"] = rel_frobenius(x2, rnd(xd + _unpack(orc, o["oproj"].out_rel, b["a"])))
    h2 = _unpack(orc, o["norm2"].out_rel, b["h2"])
    errs["norm2"] = rel_frobenius(h2, rnd(orc.rmsnorm(x2, f64(inp["g2"]), blk.eps)))
    if blk.fused:
        contract("gate_up", o["norm2"].out_rel, b["h2"], "w_gu", o["gate_up"].out_rel, b["f"], ffn, ffn // 4)
        f_rel = o["gate_up"].out_rel
    else:
        contract("gate", o["norm2"].out_rel, b["h2"], "w_gate", o["gate"].out_rel, b["gt"], ffn, ffn // 4)
        contract("up", o["norm2"].out_rel, b["h2"], "w_up", o["up"].out_rel, b["up"], ffn, ffn // 4)
        fa = _unpack(orc, o["swiglu"].out_rel, b["f"])
        errs["swiglu"] = rel_frobenius(fa, rnd(orc.swiglu(_unpack(orc, o["gate"].out_rel, b["gt"]),
                                                                     _unpack(orc, o["up"].out_rel, b["up"]))))
        f_rel = o["swiglu"].out_rel
    if blk.fused:
        contract("down_add", f_rel, b["f"], "w_down", blk.y_rel, y, dm, dm // 2, residual=x2)
        yd = _unpack(orc, blk.y_rel, y)
    else:
        contract("down", f_rel, b["f"], "w_down", o["down"].out_rel, b["dn"], dm, dm // 2)
        yd = _unpack(orc, o["add2"].out_rel, y)
        errs["add2"] = rel_frobenius(yd, rnd(x2 + _unpack(orc, o["down"].out_rel, b["dn"])))
    assert np.isfinite(yd).all()
    return errs, yd


def _chain(orc, blk, inp, yd, toks, fused, dt):
    """The oracle's own chain from the block inputs, at the listed tokens
    (all of them when toks is None), against the GPU's block output."""
    dec = _fmt(orc, dt)[0]
    f = {k: dec(v) for k, v in inp.items()}
    args = (f["x"], f["g1"], f["w_qkv"], f["w_o"], f["g2"], f["w_gate"], f["w_up"], f["w_down"], blk.batch, blk.seq,
            blk.heads)
    kw = dict(kv_heads=blk.kv_heads, fused=fused, dtype=dt)
    if toks is None:
        return rel_frobenius(yd, orc.llama_block(*args, **kw))
    return rel_frobenius(yd[toks], orc.llama_block_tokens(*args, toks, **kw))


REDUCED = [  # (name, batch, seq, dm, heads, kv_heads, ffn, seed, dtype)
    ("mha", 2, 256, 256, 2, 2, 704, 11, "bf16"),
    ("mha_f16", 2, 256, 256, 2, 2, 704, 15, "f16"),
    ("gqa", 2, 256, 1024, 8, 2, 768, 13, "bf16"),
    ("gqa_f16", 1, 384, 1024, 8, 2, 768, 16, "f16"),
]


@pytest.mark.parametrize("layout,split", [("tokens", True), ("heads", True), ("tokens", False)])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
def test_block_reduced_shapes(orc, case, fused, layout, split):
    """Every step and the whole chain compared in full (the chain at the
    per-step bar), with attention on the projections' token-major relations
    and on head-major ones (repartitions around it); at these sizes every
    contraction with two or more K tuples runs split into per-tuple partials
    and their SUM (split=True), or fused."""
    name, batch, seq, dm, heads, kv, ffn, seed, dt = case
    blk, inp, x, y = _run_block(orc, batch, seq, dm, heads, ffn, seed=seed, kv_heads=kv, fused=fused, dt=dt,
                                layout=layout, split_small=split)
    try:
        errs, yd = _check_steps(orc, blk, inp, y, sampled=False, dt=dt)
        chain = _chain(orc, blk, inp, yd, None, fused, dt)
        print("per-step errors:", {k: "%.2e" % v for k, v in errs.items()}, "chain: %.2e" % chain)
        record("block_reduced_shapes", case=name, fused=fused, layout=layout, split=sorted(blk.split), steps=errs,
               chain=chain)
        for k, v in errs.items():
            assert v <= TOL, (k, v)
        assert chain <= CHAIN_TOL
    finally:
        blk.close()


FULL = [  # (name, batch, seq, dm, heads, kv_heads, ffn, seed, dtype, sampled positions)
    # the LLaMA-7B-shaped block the bench times
    ("llama7b_4x2048", 4, 2048, 4096, 32, 32, 11008, 5, "bf16", (0, 1, 100, 500, 1000, 1500, 2047)),
    # the pages' LLaMA-3-8B-like blocks (32 query over 8 key-value heads, FFN 14,336): 8 x 1,024 tokens in
    # bf16 and in FP16 (the pages' precision), and single sequences of 1,024 and 8,192 tokens in FP16
    ("llama3_8b_8x1024", 8, 1024, 4096, 32, 8, 14336, 14, "bf16", (0, 1, 100, 511, 800, 1023)),
    ("llama3_8b_8x1024_f16", 8, 1024, 4096, 32, 8, 14336, 17, "f16", (0, 1, 100, 511, 800, 1023)),
    ("llama3_8b_1x1024_f16", 1, 1024, 4096, 32, 8, 14336, 18, "f16", (0, 1, 100, 511, 800, 1023)),
    ("llama3_8b_1x8192_f16", 1, 8192, 4096, 32, 8, 14336, 19, "f16", (0, 1, 129, 2047, 4000, 6500, 8191)),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_block_full_size(orc, case, fused):
    """Every step at full size (sampled outputs for the contractions and
    attention, full tensors otherwise, repartitions bit-exact) and the chain
    at tokens spanning each sequence."""
    name, batch, seq, dm, heads, kv, ffn, seed, dt, pos = case
    blk, inp, x, y = _run_block(orc, batch, seq, dm, heads, ffn, seed=seed, kv_heads=kv, fused=fused, dt=dt)
    try:
        errs, yd = _check_steps(orc, blk, inp, y, sampled=True, dt=dt)
        toks = [bb * seq + s for bb in sorted({0, batch // 2, batch - 1}) for s in pos]
        chain = _chain(orc, blk, inp, yd, toks, fused, dt)
        print("per-step errors:", {k: "%.2e" % v for k, v in errs.items()}, "chain: %.2e" % chain)
        record("block_full_size", case=name, fused=fused, split=sorted(blk.split), steps=errs, chain=chain,
               tokens=len(toks))
        for k, v in errs.items():
            assert v <= TOL, (k, v)
        # fp16 P costs the bf16 chain up to 5e-3 at full size; an all-half block keeps the 2e-3 bar
        assert chain <= (CHAIN_TOL if dt == "f16" else CHAIN_TOL_FULL)
    finally:
        blk.close()
