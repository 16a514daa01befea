"""Logical optimization (the pages' section 4): the oracle's exhaustive
search pinned against the pages' worked cases and hand-computed costs, then
the library's dynamic program (ja_graph_*) checked against it.  CPU only."""
import itertools

import numpy as np
import pytest

from oracle import planner as P


@pytest.fixture(scope="module")
def B():
    from tensor_relational_join_amd import binding

    return binding


# ------------------------------------------------------------------ oracle pins

def test_3d_matmul_is_optimal():
    """Section 4.4: one N x N x N matrix multiply with computation inputs on
    p = q^3 processors.  A spec with a, b, c intervals on i, j, k joins the
    first input c times over and the second a times over (N^2 (a + c)) and
    aggregates b copies of every output block ((b - 1) N^2), so the cost is
    N^2 (a + b + c - 1), least at a = b = c = q (the classical 3D algorithm)."""
    N = 48
    for q in (1, 2, 3, 4):
        g = P.Graph()
        x, y = g.input((N, N)), g.input((N, N))
        g.op("ij,jk->ik", "contract", [x, y])
        for spec in P.candidate_specs(g.ops[0], q ** 3):
            assert sum(P.plan_cost(g, [spec])) == N * N * (spec["i"] + spec["j"] + spec["k"] - 1)
        cost, plan = P.brute_force(g, q ** 3)
        assert cost == N * N * (3 * q - 1) and plan == [{"i": q, "j": q, "k": q}]


def test_example_3_8_cost_by_hand():
    """Section 3.3 / Example 3.8: i = k = 256, j = 512, i and j cut in two, k
    whole.  Four function specs, each joining a 128 x 256 block of the first
    input with a 256 x 256 block of the second: join = 4 (32,768 + 65,536) =
    393,216.  Two output types ([0,128) x [0,256) and [128,256) x [0,256)),
    each made twice: aggregation = 2 (2 - 1) 32,768 = 65,536."""
    g = P.Graph()
    a, b = g.input((256, 512)), g.input((512, 256))
    g.op("ij,jk->ik", "contract", [a, b])
    assert P.plan_cost(g, [{"i": 2, "j": 2, "k": 1}]) == (0.0, 393216.0, 65536.0)


def test_repartition_by_hand():
    """Two chained products on p = 2: the first cuts i (its output leaves
    tiling (2, 1)), the second cuts l, reading that output whole (tiling
    (1, 1)), so the 64 x 32 intermediate is repartitioned: 2,048 elements.
    The second product's own join: its (64 x 32) first input twice over and
    two 32 x 8 halves of its second input: 2 x 2,048 + 512 = 4,608."""
    g = P.Graph()
    a, b, c = g.input((64, 16)), g.input((16, 32)), g.input((32, 16))
    t = g.op("ij,jk->ik", "contract", [a, b])
    g.op("ik,kl->il", "contract", [t, c])
    rep, join, agg = P.plan_cost(g, [{"i": 2, "j": 1, "k": 1}, {"i": 1, "k": 1, "l": 2}])
    assert rep == 64 * 32
    assert join == (2 * (32 * 16 + 16 * 32)) + (2 * 64 * 32 + 2 * 32 * 8)
    assert agg == 0.0
    # the same tiling on both sides costs no repartition
    assert P.plan_cost(g, [{"i": 2, "j": 1, "k": 1}, {"i": 2, "k": 1, "l": 1}])[0] == 0.0


def test_causal_attention_joins_only_kept_tuples():
    """Causal attention with s and t cut in two keeps 3 of the 4 cells (the
    key block after the query block is dropped), so the join counts three
    (Q, K, V) block triples; each of the two output blocks of the first query
    half is made once and the second twice: aggregation = one O block."""
    g = P.Graph()
    q, k, v = g.input((1, 2, 64, 128)), g.input((1, 2, 64, 128)), g.input((1, 2, 64, 128))
    g.op("bhsd,bhtd,bhtd->bhsd", "attention", [q, k, v], "causal=s,t")
    spec = {"b": 1, "h": 1, "s": 2, "d": 1, "t": 2}
    blk = 2 * 32 * 128
    assert P.plan_cost(g, [spec]) == (0.0, 3 * 3 * blk, blk)
    assert [c for c in P.shardable(g.ops[0])] == ["b", "h", "s", "t"]


def test_pieces_of_a_residual_ffn():
    """Section 4.5 on a pre-norm FFN with a residual: the norm's output feeds
    both projections, so both edges out of it are cut (x, a computation
    input, costs nothing to share).  Pieces: the tree {gate, up, SwiGLU, down,
    add} rooted at the add, then the norm by itself."""
    g = _ffn_graph_oracle()
    ps = P.pieces(g)
    assert ps == [(5, [1, 2, 3, 4, 5]), (0, [0])]


# ------------------------------------------------------------------ graphs in both worlds

def _ffn_desc(T=64, D=32, F=48):
    """A pre-norm FFN block with its residual: norm, gate, up, SwiGLU, down,
    add.  Returns (inputs, ops) where ops are (einsum, kind, params, inputs)
    and tensor ids count inputs first, then operator outputs in order."""
    inputs = [(T, D), (D,), (D, F), (D, F), (F, D)]  # x, gain, W_gate, W_up, W_down
    x, gn, wg, wu, wd = range(5)
    n = len(inputs)
    ops = [("rd,d->rd", "rmsnorm", "eps=1e-6", [x, gn]),          # n+0
           ("td,df->tf", "contract", "", [n + 0, wg]),           # n+1
           ("td,df->tf", "contract", "", [n + 0, wu]),           # n+2
           ("rf,rf->rf", "swiglu", "", [n + 1, n + 2]),          # n+3
           ("tf,fd->td", "contract", "", [n + 3, wd]),           # n+4
           ("rd,rd->rd", "add", "", [n + 4, x])]                 # n+5
    return inputs, ops


def _view_desc():
    """A projection whose output is read head-major (a view) by an attention
    and then read back token-major (a view) by a second projection:
    y = x W1 [T, H*D]; Q = K = V = view(y) [1, H, T, D]; O = attention;
    o = view(O) [T, H*D]; z = o W2."""
    T, H, D = 16, 2, 8
    inputs = [(T, 12), (12, H * D), (H * D, 10)]
    ops = [("td,dn->tn", "contract", "", [0, 1]),                                     # 3
           ("VIEW", (1, H, T, D), ((T, H, D), (1, 0, 2)), [3]),                       # 4 (a view)
           ("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t", [4, 4, 4]),            # 5
           ("VIEW", (T, H * D), ((H, T, D), (1, 0, 2)), [5]),                         # 6 (a view)
           ("tm,mn->tn", "contract", "", [6, 2])]                                     # 7
    return inputs, ops


def _oracle_graph_v(inputs, ops):
    g = P.Graph()
    for s in inputs:
        g.input(s)
    for einsum, kind, params, ins in ops:
        if einsum == "VIEW":
            g.view(ins[0], kind)
        else:
            g.op(einsum, kind, ins, params)
    return g


def test_view_edges_cost_one_repartition_whatever_the_tilings():
    """A view is realised by a repartition into the consumer's blocking: every
    edge out of it costs all its elements (three for the attention reading
    Q, K and V from one view), under every joint choice of specs, and it
    decouples the operators around it, so the exhaustive optimum is each
    operator's cheapest join + aggregation plus those fixed charges."""
    inputs, ops = _view_desc()
    og = _oracle_graph_v(inputs, ops)
    views = 3 * 16 * 16 + 16 * 16  # three edges out of the head-major view, one out of the token-major one
    for p in (2, 4):
        cands = [P.candidate_specs(op, p) for op in og.ops]
        for plan in itertools.islice(itertools.product(*cands), 0, None, 7):
            rep, _, _ = P.plan_cost(og, plan)
            assert rep == views
        best, _ = P.brute_force(og, p)
        assert best == pytest.approx(views + sum(min(sum(P.spec_subcosts(op, c)) for c in cs)
                                                 for op, cs in zip(og.ops, cands)), rel=1e-12)
        assert P.piecewise_plan(og, p)[0] == pytest.approx(best, rel=1e-12)
        # the device model charges one copy launch per view edge on top of the operators
        plan = [cs[0] for cs in cands]
        ops_us = sum(P.op_device_time(op, c) for op, c in zip(og.ops, plan))
        assert P.plan_device_time(og, plan) == pytest.approx(
            ops_us + 4 * P.LAUNCH_US + 2 * 2 * views / P.COPY_BPS * 1e6, rel=1e-12)


def test_library_plans_graphs_with_views(B):
    """The library's planner on the graph with views: its plans (optimal,
    greedy, device) cost what the oracle says they cost, the optimum is the
    exhaustive one, and the device model agrees with the oracle's."""
    inputs, ops = _view_desc()
    og = _oracle_graph_v(inputs, ops)
    g = B.ja_graph_create()
    try:
        for sh in inputs:
            B.ja_graph_add_input(g, list(sh))
        letters = []
        for einsum, kind, params, ins in ops:
            if einsum == "VIEW":
                vshape, perm = params
                B.ja_graph_add_view(g, ins[0], B.make_view(vshape, perm), list(kind))
            else:
                sp = B.ja_spec_create(einsum, kind, params)
                letters.append(B.ja_spec_letters(sp))
                B.ja_graph_add_op(g, sp, ins)
                B.ja_spec_destroy(sp)
        assert B.ja_graph_count(g) == (3, 8)
        for p in (2, 4):
            cost = B.ja_graph_plan(g, p, B.JA_PLAN_OPTIMAL)
            plan = _lib_plan(B, g, letters)
            assert cost == pytest.approx(sum(P.plan_cost(og, plan)), rel=1e-12)
            assert cost == pytest.approx(P.brute_force(og, p)[0], rel=1e-12)
            B.ja_graph_plan(g, p, B.JA_PLAN_GREEDY)
            assert B.ja_graph_cost(g) == pytest.approx(P.plan_cost(og, _lib_plan(B, g, letters)), rel=1e-12)
            us = B.ja_graph_plan(g, p, B.JA_PLAN_DEVICE)
            assert us == pytest.approx(P.plan_device_time(og, _lib_plan(B, g, letters)), rel=1e-9)
        # a view must keep the element count and may not re-index another view
        with pytest.raises(B.JaError) as e:
            B.ja_graph_add_view(g, 3, B.make_view((16, 2, 8), (1, 0, 2)), [1, 2, 16, 4])
        assert e.value.name == "JA_ERR_SHAPE"
        with pytest.raises(B.JaError) as e:
            B.ja_graph_add_view(g, 4, B.make_view((2, 16, 8), (0, 1, 2)), [32, 8])
        assert e.value.name == "JA_ERR_UNSUPPORTED"
    finally:
        B.ja_graph_destroy(g)


def _ffn_graph_oracle():
    inputs, ops = _ffn_desc()
    return _oracle_graph(inputs, ops)


def _oracle_graph(inputs, ops):
    g = P.Graph()
    for s in inputs:
        g.input(s)
    for einsum, kind, params, ins in ops:
        g.op(einsum, kind, ins, params)
    return g


def _lib_graph(B, inputs, ops):
    g = B.ja_graph_create()
    specs = []
    for s in inputs:
        B.ja_graph_add_input(g, list(s))
    letters = []
    for einsum, kind, params, ins in ops:
        sp = B.ja_spec_create(einsum, kind, params)
        specs.append(sp)
        letters.append(B.ja_spec_letters(sp))
        B.ja_graph_add_op(g, sp, ins)
    for sp in specs:
        B.ja_spec_destroy(sp)  # the graph keeps its own copies
    return g, letters


def _lib_plan(B, g, letters):
    return [dict(zip(L, B.ja_graph_plan_intervals(g, i, len(L)))) for i, L in enumerate(letters)]


def _chain(dims):
    """M1 (M2 (... Mn)) right-associated: ops multiply from the right end."""
    inputs = [(dims[i], dims[i + 1]) for i in range(len(dims) - 1)]
    n = len(inputs)
    ops, cur = [], n - 1
    names = "abcdefgh"
    for m in range(n - 2, -1, -1):
        i, j, k = names[m], names[m + 1], names[n]
        ops.append(("%s%s,%s%s->%s%s" % (i, j, j, k, i, k), "contract", "", [m, cur]))
        cur = n + len(ops) - 1
    return inputs, ops


CHAINS = [([24, 16, 40, 8], 4), ([24, 16, 40, 8], 8), ([30, 12, 20, 18, 10], 6), ([64, 8, 64, 8], 8),
          ([16, 48, 16, 48, 16], 4)]


@pytest.mark.parametrize("dims,p", CHAINS)
def test_dynamic_program_is_optimal_on_trees(B, dims, p):
    """A matrix chain is a tree: the library's dynamic program reaches the
    exhaustive minimum, and its reported cost is the oracle's cost of the
    plan it returns."""
    inputs, ops = _chain(dims)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        cost = B.ja_graph_plan(g, p, B.JA_PLAN_OPTIMAL)
        plan = _lib_plan(B, g, letters)
        og = _oracle_graph(inputs, ops)
        assert cost == pytest.approx(sum(P.plan_cost(og, plan)), rel=1e-12)
        assert cost == pytest.approx(P.brute_force(og, p)[0], rel=1e-12)
        assert B.ja_graph_cost(g) == pytest.approx(P.plan_cost(og, plan), rel=1e-12)
    finally:
        B.ja_graph_destroy(g)


@pytest.mark.parametrize("dims,p", CHAINS[:3])
def test_greedy_and_random_selectors(B, dims, p):
    """Greedy (section 6, Experiment 3): the same program without the
    repartition sub-cost, so every operator takes its cheapest join +
    aggregation and the plan costs at least the optimum.  Random: a valid spec
    per operator, costed like any plan."""
    inputs, ops = _chain(dims)
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        opt = B.ja_graph_plan(g, p, B.JA_PLAN_OPTIMAL)
        greedy = B.ja_graph_plan(g, p, B.JA_PLAN_GREEDY)
        plan = _lib_plan(B, g, letters)
        _, j, a = P.plan_cost(og, plan)
        assert j + a == pytest.approx(sum(min(sum(P.spec_subcosts(op, c)) for c in P.candidate_specs(op, p))
                                          for op in og.ops), rel=1e-12)
        assert greedy >= opt - 1e-9
        for seed in range(5):
            c = B.ja_graph_plan(g, p, B.JA_PLAN_RANDOM, seed)
            plan = _lib_plan(B, g, letters)
            for spec in plan:
                assert int(np.prod(list(spec.values()))) == p
            assert c == pytest.approx(sum(P.plan_cost(og, plan)), rel=1e-12)
            assert c >= opt - 1e-9
    finally:
        B.ja_graph_destroy(g)


@pytest.mark.parametrize("p", [2, 4, 8])
def test_pieces_are_planned_optimally(B, p):
    """A graph that is not a tree (the residual FFN): every piece of the
    library's plan is the exhaustive optimum given the pieces planned before
    it (section 4.5's guarantee), and the reported cost is the plan's cost."""
    inputs, ops = _ffn_desc()
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        cost = B.ja_graph_plan(g, p, B.JA_PLAN_OPTIMAL)
        plan = _lib_plan(B, g, letters)
        assert cost == pytest.approx(sum(P.plan_cost(og, plan)), rel=1e-12)
        fixed = [None] * len(og.ops)
        for root, piece in P.pieces(og):
            for i in piece:
                fixed[i] = plan[i]
            best, _ = P.best_piece(og, p, [f if (k not in piece) else None for k, f in enumerate(fixed)],
                                   root, piece)
            assert P.piece_cost(og, fixed, root, piece) == pytest.approx(best, rel=1e-12)
    finally:
        B.ja_graph_destroy(g)


def test_library_recovers_the_3d_algorithm(B):
    g, letters = _lib_graph(B, [(96, 96), (96, 96)], [("ij,jk->ik", "contract", "", [0, 1])])
    try:
        for q in (2, 3, 4):
            cost = B.ja_graph_plan(g, q ** 3)
            assert cost == 96 * 96 * (3 * q - 1)
            assert B.ja_graph_plan_intervals(g, 0, 3) == [q, q, q]
    finally:
        B.ja_graph_destroy(g)


def test_attention_and_norm_costs_match_oracle(B):
    """Causal attention (only kept tuples join) and RMSNorm (per-row sums
    aggregated over feature intervals) cost the same in both worlds for every
    candidate the planner would consider."""
    inputs = [(2, 4, 96, 128)] * 3 + [(96, 64), (64,)]
    ops = [("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t", [0, 1, 2]),
           ("rd,d->rd", "rmsnorm", "eps=1e-6", [3, 4])]
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        for p in (4, 6, 8):
            for sa in P.candidate_specs(og.ops[0], p):
                for sn in P.candidate_specs(og.ops[1], p):
                    iv = [[sa[c] for c in letters[0]], [sn[c] for c in letters[1]]]
                    assert B.ja_graph_cost(g, iv) == pytest.approx(P.plan_cost(og, [sa, sn]), rel=1e-12)
            cost = B.ja_graph_plan(g, p)
            assert cost == pytest.approx(P.brute_force(og, p)[0], rel=1e-12)
    finally:
        B.ja_graph_destroy(g)


def test_planner_errors(B):
    g = B.ja_graph_create()
    try:
        x = B.ja_graph_add_input(g, [4, 3])
        y = B.ja_graph_add_input(g, [5, 2])
        s = B.ja_spec_create("ij,jk->ik", "contract", "")
        with pytest.raises(B.JaError) as e:  # j would be both 3 and 5
            B.ja_graph_add_op(g, s, [x, y])
        assert e.value.name == "JA_ERR_SHAPE"
        y = B.ja_graph_add_input(g, [3, 2])
        B.ja_graph_add_op(g, s, [x, y])
        B.ja_spec_destroy(s)
        with pytest.raises(B.JaError) as e:  # 4 * 3 * 2 = 24 cells at most
            B.ja_graph_plan(g, 25)
        assert e.value.name == "JA_ERR_UNSUPPORTED"
        with pytest.raises(B.JaError) as e:
            B.ja_graph_plan_intervals(g, 0, 3)
        assert e.value.name == "JA_ERR_STATE"
        sp = B.ja_spec_create("bhsd,bhtd,bhtd->bhsd", "attention", "packed=8,16")
        q = B.ja_graph_add_input(g, [1, 1, 16, 128])
        with pytest.raises(B.JaError) as e:
            B.ja_graph_add_op(g, sp, [q, q, q])
        assert e.value.name == "JA_ERR_UNSUPPORTED"
        B.ja_spec_destroy(sp)
    finally:
        B.ja_graph_destroy(g)


# ------------------------------------------------------------------ device-time model

def test_device_model_closed_forms():
    """The model's arithmetic on cases whose answer is known: 256 equal tiles
    fill the 256 CUs once, one tile more takes a second round (a contraction
    runs a last round of at most 128 tiles as half-height tiles); a 4,096^3
    product as one block is 16 x 16 tiles of K = 4,096; a copy-bound
    operator is its bytes over the copy rate."""
    assert P.makespan([1.0] * 256) == 1.0 and P.makespan([1.0] * 257) == 2.0
    assert P.makespan([3.0, 2.0, 2.0, 1.0], cus=2) == 4.0  # 3+1 and 2+2
    g = P.Graph()
    a, b = g.input((4096, 4096)), g.input((4096, 4096))
    g.op("ij,jk->ik", "contract", [a, b])
    tile = 2.0 * 256 * 256 * 4096 / P.GEMM_CU_FLOPS * 1e6
    assert P.op_device_time(g.ops[0], {"i": 1, "j": 1, "k": 1}) == pytest.approx(P.LAUNCH_US + tile)
    # j cut in two: each output tile still does all 4,096 contracted elements (the SUM is fused)
    assert P.op_device_time(g.ops[0], {"i": 1, "j": 2, "k": 1}) == pytest.approx(P.LAUNCH_US + tile)
    # i cut in 8 x 512-row blocks: 2 x 16 tiles per block, 256 tiles in all, one round
    assert P.op_device_time(g.ops[0], {"i": 8, "j": 1, "k": 1}) == pytest.approx(P.LAUNCH_US + tile)
    # i cut in 3: 1,366 / 1,365-row blocks give 6 x 16 tiles each (288 > 256): one full round, then the other
    # 32 tiles as 64 half-height tiles in a second launch
    assert P.op_device_time(g.ops[0], {"i": 3, "j": 1, "k": 1}) == pytest.approx(
        2 * P.LAUNCH_US + tile + P.HALF_TILE * tile)
    # i cut in 25: 163 / 164-row blocks of 1 x 16 tiles, 400 in all: the last round (144) would fill more than
    # half the CUs, so it runs at full height: two rounds
    assert P.op_device_time(g.ops[0], {"i": 25, "j": 1, "k": 1}) == pytest.approx(P.LAUNCH_US + 2 * tile)
    assert P.contract_makespan([1.0] * 512) == 2.0  # whole rounds: no second launch
    g2 = P.Graph()
    x, y = g2.input((1024, 4096)), g2.input((1024, 4096))
    g2.op("rd,rd->rd", "add", [x, y])
    assert P.op_device_time(g2.ops[0], {"r": 2, "d": 4}) == pytest.approx(
        P.LAUNCH_US + 6.0 * 1024 * 4096 / P.COPY_BPS * 1e6)


def test_device_model_tail_matches_oracle(B):
    """Library and oracle agree where a contraction's last round runs as
    half-height tiles (288 tiles), where it does not (400), and on whole
    rounds (256)."""
    inputs = [(4096, 4096), (4096, 4096)]
    ops = [("ij,jk->ik", "contract", "", [0, 1])]
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        for i in (3, 25, 8):
            sp = {"i": i, "j": 1, "k": 1}
            iv = [[sp[c] for c in letters[0]]]
            assert B.ja_graph_device_time(g, iv) == pytest.approx(P.plan_device_time(og, [sp]), rel=1e-9)
    finally:
        B.ja_graph_destroy(g)


@pytest.mark.parametrize("dims,p", CHAINS[:3])
def test_device_model_matches_oracle(B, dims, p):
    """Library and oracle compute the same modelled time for every plan of a
    chain, and the library's JA_PLAN_DEVICE reaches the exhaustive minimum."""
    inputs, ops = _chain([d * 64 for d in dims])
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        cands = [P.candidate_specs(op, p) for op in og.ops]
        for plan in list(itertools.product(*cands))[::7]:
            iv = [[sp[c] for c in L] for sp, L in zip(plan, letters)]
            assert B.ja_graph_device_time(g, iv) == pytest.approx(P.plan_device_time(og, plan), rel=1e-9)
        t = B.ja_graph_plan(g, p, B.JA_PLAN_DEVICE)
        assert t == pytest.approx(P.brute_force_device(og, p), rel=1e-9)
        assert t == pytest.approx(P.plan_device_time(og, _lib_plan(B, g, letters)), rel=1e-9)
    finally:
        B.ja_graph_destroy(g)


def test_device_model_attention_and_ffn(B):
    """Causal attention tiles see only the keys up to their last row; the
    residual FFN (not a tree) is planned piece by piece like the proxy."""
    inputs = [(2, 8, 1024, 128)] * 3
    ops = [("bhsd,bhtd,bhtd->bhsd", "attention", "causal=s,t", [0, 1, 2])]
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        for spec in P.candidate_specs(og.ops[0], 8):
            iv = [[spec[c] for c in letters[0]]]
            assert B.ja_graph_device_time(g, iv) == pytest.approx(P.plan_device_time(og, [spec]), rel=1e-9)
    finally:
        B.ja_graph_destroy(g)
    inputs, ops = _ffn_desc(T=2048, D=1024, F=2816)
    og = _oracle_graph(inputs, ops)
    g, letters = _lib_graph(B, inputs, ops)
    try:
        t = B.ja_graph_plan(g, 8, B.JA_PLAN_DEVICE)
        assert t == pytest.approx(P.plan_device_time(og, _lib_plan(B, g, letters)), rel=1e-9)
        assert t == pytest.approx(B.ja_graph_device_time(g), rel=1e-12)
    finally:
        B.ja_graph_destroy(g)
