"""GPU parity of planned computation graphs (graph.Graph / PlannedRun):
whatever join-agg spec the logical optimizer (or the greedy or random
selector) picks per operator, running the plan on the GPU -- operators with
those decompositions, computation inputs materialised in their consumers'
blockings, repartitions on the edges whose blockings differ -- gives every
operator's output within the bf16 bar of the oracle applied to that
operator's own inputs."""
import numpy as np
import pytest

from gpu_helpers import bf16_bits, rel_frobenius

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3


@pytest.fixture(scope="module")
def G():
    import torch

    assert torch.cuda.is_available()
    from tensor_relational_join_amd import graph

    return graph


def _dense_bits(t):
    return bf16_bits(t.contiguous().view(-1)).reshape(tuple(t.shape))


def _oracle_step(orc, op, ins):
    f = [orc.bf16_to_f64(x) for x in ins]
    if op["kind"] == "contract":
        return orc.einsum(op["einsum"], f[0], f[1])
    if op["kind"] == "rmsnorm":
        return orc.rmsnorm(f[0], f[1], 1e-6)
    if op["kind"] == "swiglu":
        return orc.swiglu(f[0], f[1])
    return orc.add(f[0], f[1])


def _check_plan(G, orc, g, plan, inputs):
    import torch

    run = G.PlannedRun(g, plan)
    try:
        run.load(inputs)
        run.run()
        torch.cuda.synchronize()
        dense = dict((t, _dense_bits(x)) for t, x in inputs.items())
        for i, op in enumerate(g.ops):
            dense[g.producer.index(i)] = _dense_bits(run.dense_output(i))
        for i, op in enumerate(g.ops):
            want = orc.round_bf16(_oracle_step(orc, op, [dense[t] for t in op["inputs"]]))
            got = orc.bf16_to_f64(dense[g.producer.index(i)])
            assert rel_frobenius(got, want) <= BF16_TOL, (i, op["einsum"], plan[i])
        return len(run.reparts)
    finally:
        run.close()


def _inputs(g, seed, stds):
    import torch

    torch.manual_seed(seed)
    return {t: torch.empty(g.shapes[t], dtype=torch.bfloat16, device="cuda").normal_(m, s)
            for t, (m, s) in stds.items()}


def test_chain_under_every_selector(G, orc):
    """A right-associated four-matrix chain, M1 (M2 (M3 M4)), on p = 8: the
    optimizer's, the greedy and five random plans."""
    from tensor_relational_join_amd.binding import JA_PLAN_GREEDY, JA_PLAN_OPTIMAL, JA_PLAN_RANDOM

    g = G.Graph()
    m = [g.input(s) for s in ((256, 512), (512, 384), (384, 640), (640, 128))]
    x = g.op("cd,de->ce", "contract", [m[2], m[3]])
    y = g.op("bc,ce->be", "contract", [m[1], x])
    g.op("ab,be->ae", "contract", [m[0], y])
    inputs = _inputs(g, 7, {t: (0.0, 0.05) for t in m})
    nrep = []
    for mode, seed in [(JA_PLAN_OPTIMAL, 0), (JA_PLAN_GREEDY, 0)] + [(JA_PLAN_RANDOM, s) for s in range(5)]:
        cost, plan = g.plan(8, mode, seed)
        nrep.append(_check_plan(G, orc, g, plan, inputs))
    assert max(nrep) > 0  # some plan repartitions between operators


def test_residual_ffn_plans(G, orc):
    """The pre-norm FFN with its residual (a graph that is not a tree): norm,
    gate, up, SwiGLU, down, add, on p = 8 and p = 4."""
    from tensor_relational_join_amd.binding import JA_PLAN_OPTIMAL, JA_PLAN_RANDOM

    T, D, F = 512, 256, 704
    g = G.Graph()
    x, gn, wg, wu, wd = g.input((T, D)), g.input((D,)), g.input((D, F)), g.input((D, F)), g.input((F, D))
    h = g.op("rd,d->rd", "rmsnorm", [x, gn], "eps=1e-6")
    a = g.op("td,df->tf", "contract", [h, wg])
    b = g.op("td,df->tf", "contract", [h, wu])
    s = g.op("rf,rf->rf", "swiglu", [a, b])
    dn = g.op("tf,fd->td", "contract", [s, wd])
    g.op("rd,rd->rd", "add", [dn, x])
    inputs = _inputs(g, 8, {x: (0.0, 1.0), gn: (1.0, 0.1), wg: (0.0, 0.05), wu: (0.0, 0.05), wd: (0.0, 0.05)})
    for p in (8, 4):
        for mode, seed in [(JA_PLAN_OPTIMAL, 0), (JA_PLAN_RANDOM, 1), (JA_PLAN_RANDOM, 2)]:
            _, plan = g.plan(p, mode, seed)
            _check_plan(G, orc, g, plan, inputs)


def test_llama_block_graph_plans(G, orc):
    """The LLaMA-shaped block as a graph of the pages' operators with views
    between the token-major projections and the head-major attention
    (graph.llama_block_graph), planned on p = 8 by the optimizer, the greedy
    selector, the device-time model and a random choice, and under the
    LlamaBlock class's hand decompositions: every plan's block output
    against the oracle's own block (Q, K and V as the column groups of one
    fused projection: the same values, rounded at the same points) end to
    end, at reduced shapes."""
    import torch

    from tensor_relational_join_amd import synth
    from tensor_relational_join_amd.binding import JA_PLAN_DEVICE, JA_PLAN_GREEDY, JA_PLAN_OPTIMAL, JA_PLAN_RANDOM

    batch, seq, dm, heads, ffn = 2, 256, 256, 2, 704
    g, t = G.llama_block_graph(batch, seq, dm, heads, ffn)
    inp = synth.llama_block_inputs(21, batch, seq, dm, ffn)
    w = dict(inp)
    for i, n in enumerate("qkv"):
        w["w_" + n] = np.ascontiguousarray(inp["w_qkv"][:, i * dm:(i + 1) * dm])
    dev = {t[n]: torch.from_numpy(np.ascontiguousarray(w[n]).view(np.int16)).view(torch.bfloat16).cuda()
           for n in ("x", "g1", "w_q", "w_k", "w_v", "w_o", "g2", "w_gate", "w_up", "w_down")}
    f = {k: orc.bf16_to_f64(v) for k, v in inp.items()}
    want = orc.llama_block(f["x"], f["g1"], f["w_qkv"], f["w_o"], f["g2"], f["w_gate"], f["w_up"], f["w_down"],
                           batch, seq, heads)
    y_op = g.producer[t["y"]]
    runs = [(mode, seed, None) for mode, seed in ((JA_PLAN_OPTIMAL, 0), (JA_PLAN_GREEDY, 0), (JA_PLAN_DEVICE, 0),
                                                  (JA_PLAN_RANDOM, 3))]
    runs.append((None, 0, G.llama_block_hand_splits(g, batch, seq)))
    for mode, seed, splits in runs:
        plan = g.plan(8, mode, seed)[1] if splits is None else None
        run = G.PlannedRun(g, plan, splits=splits)
        try:
            run.load(dev)
            run.run()
            torch.cuda.synchronize()
            got = orc.bf16_to_f64(_dense_bits(run.dense_output(y_op)))
        finally:
            run.close()
        assert rel_frobenius(got, want) <= BF16_TOL, (mode, seed, splits is not None)
