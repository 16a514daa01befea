"""GPU parity of attention planned on the device (ja_dattn_*, spec
"packed=device"): sequence ends drawn on the GPU are the split points of the
sequence letters; the device-side join, the table-building kernels and the
attention kernel run with no host round trip.  Checked against the oracle's
packed attention, bit for bit against the host-planned packed path on the
same cuts, and for bad split points (a status word, O untouched)."""
import numpy as np
import pytest

from gpu_helpers import bf16_bits, rel_frobenius

pytestmark = pytest.mark.gpu

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


def _draw_ends(S, nseq, seed):
    """nseq sequence ends in (0, S], the last at S, drawn on the GPU."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    cuts = torch.randperm(S - 1, generator=g, device="cuda")[: nseq - 1] + 1
    return torch.cat([torch.zeros(1, dtype=torch.int64, device="cuda"), cuts.sort().values,
                      torch.full((1,), S, dtype=torch.int64, device="cuda")])


def _case(dev, orc, G, R, S, nseq, gint, causal, seed):
    import torch

    einsum = "bgrsd,bgtd,bgtd->bgrsd"  # letters b g r s d t
    params = "packed=device" + (";causal=s,t" if causal else "")
    counts = {"b": 1, "g": gint, "r": 1, "s": nseq, "d": 1, "t": nseq}
    extents = {"b": 1, "g": G, "r": R, "s": S, "d": 128, "t": S}
    da = dev.DeviceAttention(einsum, counts, extents, params)
    try:
        gen = torch.Generator(device="cuda").manual_seed(seed)
        Q = torch.empty(G * R * S * 128, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
        K = torch.empty(G * S * 128, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
        V = torch.empty(G * S * 128, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
        O = torch.full_like(Q, 7.0)
        ends = _draw_ends(S, nseq, seed)
        d = lambda lo, hi: torch.tensor([lo, hi], dtype=torch.int64, device="cuda")  # noqa: E731
        gsp = torch.tensor(_eq(G, gint), dtype=torch.int64, device="cuda")
        splits = torch.cat([d(0, 1), gsp, d(0, R), ends, d(0, 128), ends])
        da.run(splits, Q, K, V, O)
        torch.cuda.synchronize()
        nt, ns, status = (int(x) for x in da.counts.cpu())
        e = ends.cpu().tolist()
    finally:
        da.close()
    # Q, O blocked by b, g, r only: g-blocks of [1, g, R, S, 128] back to back
    q_rel = orc.Relation((1, G, R, S, 128), [[0, 1], _eq(G, gint), [0, R], [0, S], [0, 128]])
    k_rel = orc.Relation((1, G, S, 128), [[0, 1], _eq(G, gint), [0, S], [0, 128]])
    host = dict(Q=q_rel.unpack(bf16_bits(Q)), K=k_rel.unpack(bf16_bits(K)), V=k_rel.unpack(bf16_bits(V)),
                O=q_rel.unpack(bf16_bits(O)))
    return host, e, (nt, ns, status)


@pytest.mark.parametrize("G,R,S,nseq,gint,causal", [
    (2, 4, 3000, 7, 1, True),     # grouped-query, causal, ragged sequences
    (4, 1, 2048, 16, 2, True),    # multi-head, two head blocks
    (2, 2, 1500, 5, 2, False),    # bidirectional
    (1, 1, 700, 1, 1, True),      # one sequence: plain causal attention
])
def test_device_planned_varlen_attention(dev, orc, G, R, S, nseq, gint, causal):
    host, ends, (nt, ns, status) = _case(dev, orc, G, R, S, nseq, gint, causal, seed=21 + nseq)
    assert status == 0 and ns == gint * nseq and nt == gint * nseq  # one tuple per (head block, sequence)
    want = orc.attention(orc.bf16_to_f64(host["Q"]).reshape(1, G * R, S, 128), orc.bf16_to_f64(host["K"]),
                         orc.bf16_to_f64(host["V"]), 1.0 / np.sqrt(128.0), causal, seq_ends=ends[1:])
    got = orc.bf16_to_f64(host["O"]).reshape(1, G * R, S, 128)
    assert rel_frobenius(got, orc.round_bf16(want)) <= BF16_TOL


def test_device_plan_equals_host_plan_bitwise(dev, orc):
    """The same cuts planned on the host (packed=device through ja_plan_*)
    compute the same bits: every tile does the same arithmetic in the same
    order whichever side built its tables."""
    import torch

    G, R, S, nseq = 2, 4, 2500, 6
    host, ends, _ = _case(dev, orc, G, R, S, nseq, 1, True, seed=5)
    sp = {"b": [0, 1], "g": [0, G], "r": [0, R], "s": ends, "d": [0, 128], "t": ends}
    op = dev.Op("bgrsd,bgtd,bgtd->bgrsd", "attention", sp, "packed=device;causal=s,t")
    try:
        rels = op.in_rels + [op.out_rel]
        bufs = []
        for rel, key in zip(rels[:3], ("Q", "K", "V")):
            flat = orc.Relation(rel.shape, rel.splits).pack(host[key])
            bufs.append(torch.from_numpy(np.ascontiguousarray(flat).view(np.int16)).view(torch.bfloat16).cuda())
        out = dev.alloc(op.out_rel)
        op.run(bufs, out)
        torch.cuda.synchronize()
        o_host = orc.Relation(op.out_rel.shape, op.out_rel.splits).unpack(bf16_bits(out))
    finally:
        op.close()
    assert np.array_equal(o_host, host["O"])


def test_device_plan_bad_cuts_leave_output_alone(dev):
    """s and t cut differently, or cuts that are not a tiling: the status
    word says so and O keeps its contents."""
    import torch

    da = dev.DeviceAttention("bhsd,bhtd,bhtd->bhsd", {"b": 1, "h": 1, "s": 3, "d": 1, "t": 3},
                             {"b": 1, "h": 2, "s": 600, "d": 128, "t": 600})
    try:
        Q = torch.zeros(2 * 600 * 128, dtype=torch.bfloat16, device="cuda")
        O = torch.full_like(Q, 3.0)
        t = lambda v: torch.tensor(v, dtype=torch.int64, device="cuda")  # noqa: E731
        for sp, bits in (([0, 1, 0, 2, 0, 100, 300, 600, 0, 128, 0, 100, 350, 600], 4),   # s, t differ
                         ([0, 1, 0, 2, 0, 300, 100, 600, 0, 128, 0, 300, 100, 600], 1)):  # not rising
            da.run(t(sp), Q, Q, Q, O)
            torch.cuda.synchronize()
            nt, ns, status = (int(x) for x in da.counts.cpu())
            assert status & bits and nt == 0 and ns == 0
            assert bool((O == 3.0).all())
    finally:
        da.close()
