"""Logical optimization by exhaustive search -- TEST INFRASTRUCTURE ONLY
(part of the CPU oracle; the same import rules hold).

Source: "Every Kernel Is a Join: Automatic Multi-GPU Parallelism for AI
Computations in Einsummable" (paperpeel full text), section 3.3 (shardable
indices, one function spec per combination of intervals), section 4.2 (a
computation graph; choosing one join-agg spec per operator), section 4.3 (the
communication-cost proxy and its three sub-costs), section 4.4 (the 3D matrix
multiply the optimizer recovers), section 4.5 (graphs that are not trees are
cut at the edges out of multiply-consumed tensors and the pieces planned one
at a time, larger first).

Every function here enumerates: the candidate specs of an operator, the cells
of its interval grid, and every joint choice of specs.  Nothing is shared with
the library's planner.

A view (a tensor re-indexed by a reshape and a permutation of axes, e.g.
token-major projections read as head-major attention inputs) is realised by
a repartition that moves every element into whatever blocking its consumer
asks for: it is charged as a repartition on every edge out of it (all its
elements; one copy launch in the device-time model) and leaves both its
source's and its consumer's tilings free.

Readings (also in the design notes): candidate specs cut the shardable
indices into near-equal intervals whose counts multiply to p; a tiling is the
interval count per dimension; the join sub-cost counts only cells that the
causal predicate keeps; the aggregated types are the output blocks of a
contraction or attention and the per-row sums of squares of RMSNorm; edges
between pieces are charged when the second of their two pieces is planned;
pieces of equal size go in the order of their root operators.
"""
from __future__ import annotations

import itertools
from typing import Dict, List, Optional, Sequence, Tuple

from . import equal_splits


class Graph:
    """Tensors (computation inputs or operator outputs) and operators, each
    operator an einsum over named indices with an op kind and params."""

    def __init__(self):
        self.shapes: List[Tuple[int, ...]] = []
        self.producer: List[Optional[int]] = []
        self.ops: List[dict] = []
        self.view_of: Dict[int, int] = {}  # view tensor -> the tensor it re-indexes

    def input(self, shape) -> int:
        self.shapes.append(tuple(shape))
        self.producer.append(None)
        return len(self.shapes) - 1

    def op(self, einsum: str, kind: str, inputs: Sequence[int], params: str = "") -> int:
        lhs, out = einsum.split("->")
        ins = lhs.split(",")
        letters: List[str] = []
        for s in ins + [out]:
            for c in s:
                if c not in letters:
                    letters.append(c)
        ext: Dict[str, int] = {}
        for s, t in zip(ins, inputs):
            for c, e in zip(s, self.shapes[t]):
                assert ext.setdefault(c, e) == e
        causal = None
        for kv in params.split(";"):
            if kv.startswith("causal="):
                causal = tuple(kv[len("causal="):].split(","))
        self.ops.append(dict(ins=ins, out=out, kind=kind, inputs=list(inputs), letters=letters, ext=ext,
                             causal=causal))
        self.shapes.append(tuple(ext[c] for c in out))
        self.producer.append(len(self.ops) - 1)
        return len(self.shapes) - 1

    def view(self, t: int, shape) -> int:
        """Tensor t read as `shape` (same element count) after a reshape and
        a permutation of axes; which ones does not change any cost."""
        n = 1
        for e in shape:
            n *= e
        assert n == self.numel(t) and t not in self.view_of
        self.shapes.append(tuple(shape))
        self.producer.append(None)
        self.view_of[len(self.shapes) - 1] = t
        return len(self.shapes) - 1

    def consumers(self, t: int) -> List[Tuple[int, int]]:
        return [(i, k) for i, o in enumerate(self.ops) for k, x in enumerate(o["inputs"]) if x == t]

    def numel(self, t: int) -> int:
        n = 1
        for e in self.shapes[t]:
            n *= e
        return n


def shardable(op: dict) -> List[str]:
    """Section 3.3: contraction and elementwise indices are all shardable
    ("any"); attention shards the key-value batch / head indices and the
    sequence (the query-head group and the head dimension are not directly
    shardable); RMSNorm shards rows and features."""
    if op["kind"] == "attention":
        q, k = op["ins"][0], op["ins"][1]
        return [c for c in op["letters"] if (c in k or c == q[-2]) and c != q[-1]]
    return list(op["letters"])


def candidate_specs(op: dict, p: int) -> List[Dict[str, int]]:
    """Every choice of interval counts, one per shardable index (1 for the
    others), whose product is p."""
    sh = shardable(op)
    ranges = [range(1, min(op["ext"][c], p) + 1) if c in sh else range(1, 2) for c in op["letters"]]
    out = []
    for combo in itertools.product(*ranges):
        prod = 1
        for v in combo:
            prod *= v
        if prod == p:
            out.append(dict(zip(op["letters"], combo)))
    return out


def spec_subcosts(op: dict, counts: Dict[str, int]) -> Tuple[float, float]:
    """(join, aggregation) of section 4.3 for the join-agg spec with these
    interval counts: its function specifications are the cells of the
    interval grid that the join keeps."""
    sp = {c: equal_splits(op["ext"][c], counts[c]) for c in op["letters"]}
    join = 0.0
    copies: Dict[tuple, List[float]] = {}
    for cell in itertools.product(*[range(counts[c]) for c in op["letters"]]):
        at = dict(zip(op["letters"], cell))
        if op["causal"] is not None:
            s, t = op["causal"]
            if sp[t][at[t]] >= sp[s][at[s] + 1]:
                continue
        size = lambda c: sp[c][at[c] + 1] - sp[c][at[c]]  # noqa: E731
        for s in op["ins"]:
            n = 1
            for c in s:
                n *= size(c)
            join += n
        if op["kind"] in ("contract", "attention", "rmsnorm"):
            agg_letters = op["out"][:1] if op["kind"] == "rmsnorm" else op["out"]
            n = 1
            for c in agg_letters:
                n *= size(c)
            key = tuple(at[c] for c in agg_letters)
            copies.setdefault(key, []).append(n)
    agg = sum((len(v) - 1) * v[0] for v in copies.values())
    return join, agg


def tiling(letters: str, counts: Dict[str, int]) -> Tuple[int, ...]:
    return tuple(counts[c] for c in letters)


def plan_cost(g: Graph, plan: Sequence[Dict[str, int]]) -> Tuple[float, float, float]:
    """(repartition, join, aggregation) of a full assignment (section 4.3):
    an operator-produced input whose tiling under the consumer's spec differs
    from its tiling under the producer's spec costs all its elements."""
    rep = join = agg = 0.0
    for i, op in enumerate(g.ops):
        j, a = spec_subcosts(op, plan[i])
        join += j
        agg += a
        for s, t in zip(op["ins"], op["inputs"]):
            q = g.producer[t]
            if t in g.view_of:
                rep += g.numel(t)
            elif q is not None and tiling(s, plan[i]) != tiling(g.ops[q]["out"], plan[q]):
                rep += g.numel(t)
    return rep, join, agg


def brute_force(g: Graph, p: int) -> Tuple[float, List[Dict[str, int]]]:
    """The cheapest full assignment by trying every joint choice of specs."""
    cands = [candidate_specs(op, p) for op in g.ops]
    best = None
    for plan in itertools.product(*cands):
        c = sum(plan_cost(g, plan))
        if best is None or c < best[0]:
            best = (c, list(plan))
    return best


def output_tensor(g: Graph, i: int) -> int:
    return g.producer.index(i)


def pieces(g: Graph) -> List[Tuple[int, List[int]]]:
    """Section 4.5: cut every edge out of a tensor with several consumers;
    the pieces (connected by the remaining edges) as (root, operators), larger
    first, equal sizes by root.  The root is the operator whose output is not
    consumed inside its piece."""
    n = len(g.ops)
    cut = {t for t in range(len(g.shapes)) if len(g.consumers(t)) > 1}
    comp = list(range(n))

    def find(x):
        while comp[x] != x:
            x = comp[x]
        return x

    for i, op in enumerate(g.ops):
        for t in op["inputs"]:
            q = g.producer[t]
            if q is not None and t not in cut:
                comp[find(i)] = find(q)
    groups: Dict[int, List[int]] = {}
    for i in range(n):
        groups.setdefault(find(i), []).append(i)
    out = []
    for ops in groups.values():
        root = [i for i in ops if len(g.consumers(output_tensor(g, i))) != 1]
        out.append((root[0], sorted(ops)))
    out.sort(key=lambda r: (-len(r[1]), r[0]))
    return out


def piece_cost(g: Graph, plan: Sequence[Optional[Dict[str, int]]], root: int, ops: Sequence[int],
               with_repartition: bool = True) -> float:
    """What planning one piece minimizes, given `plan` (its own operators'
    specs, and those of the pieces planned before it; None elsewhere): the
    join and aggregation of its operators, and the repartitions on every edge
    whose two ends are both planned and of which at least one end is in the
    piece."""
    cost = 0.0
    for i in ops:
        op = g.ops[i]
        j, a = spec_subcosts(op, plan[i])
        cost += j + a
        if not with_repartition:
            continue
        for s, t in zip(op["ins"], op["inputs"]):
            q = g.producer[t]
            if t in g.view_of:
                cost += g.numel(t)  # a view: one repartition whatever the tilings
                continue
            if q is None or plan[q] is None:
                continue  # a computation input, or charged when the producer's piece is planned
            if tiling(s, plan[i]) != tiling(g.ops[q]["out"], plan[q]):
                cost += g.numel(t)
    if with_repartition:
        t_out = output_tensor(g, root)
        for (c, k) in g.consumers(t_out):
            if c not in ops and plan[c] is not None and \
                    tiling(g.ops[c]["ins"][k], plan[c]) != tiling(g.ops[root]["out"], plan[root]):
                cost += g.numel(t_out)
    return cost


def best_piece(g: Graph, p: int, plan: Sequence[Optional[Dict[str, int]]], root: int, ops: Sequence[int],
               with_repartition: bool = True) -> Tuple[float, List[Dict[str, int]]]:
    """The cheapest choice of specs for one piece by trying every one."""
    best = None
    for choice in itertools.product(*[candidate_specs(g.ops[i], p) for i in ops]):
        trial = list(plan)
        for i, c in zip(ops, choice):
            trial[i] = c
        cost = piece_cost(g, trial, root, ops, with_repartition)
        if best is None or cost < best[0]:
            best = (cost, list(choice))
    return best


def piecewise_plan(g: Graph, p: int, with_repartition: bool = True) -> Tuple[float, List[Dict[str, int]]]:
    """Plan the pieces one at a time (section 4.5), each by exhaustive search
    given the specs already fixed; with_repartition False charges no
    repartition while choosing (the greedy selector of section 6, Experiment
    3).  Returns the plan's full proxy cost and the plan."""
    plan: List[Optional[Dict[str, int]]] = [None] * len(g.ops)
    for root, ops in pieces(g):
        _, choice = best_piece(g, p, plan, root, ops, with_repartition)
        for i, c in zip(ops, choice):
            plan[i] = c
    return sum(plan_cost(g, plan)), plan


# --------------------------------------------------------------------------
# the device-time model of one MI355X running this library's kernels (the
# computation awareness the pages leave as future work, section 8)
#
# PARITY UNPINNED as a model of the hardware.  The pages define no such
# model: this one is written out from the library's own kernel design (tile
# shapes, the half-height last round) with rates measured on those kernels,
# and it changes with them.  Its closed-form tests pin only its arithmetic
# (rounds, placement, cuts), so it checks that the library's dynamic program
# finds the plan this model ranks best, not that the model predicts the GPU.
# --------------------------------------------------------------------------

CUS = 256
GEMM_CU_FLOPS = 1213e12 / CUS   # measured fused bf16 contraction, per CU
ATTN_CU_FLOPS = 775e12 / CUS    # measured causal attention, per CU
COPY_BPS = 5.0e12               # measured plain device copy
LAUNCH_US = 4.0
HALF_TILE = 0.66                # measured: a half-height contraction tile's time over a full tile's


def makespan(times: Sequence[float], cus: int = CUS) -> float:
    """Longest job first, each onto the CU that frees up first; the time the
    last CU finishes."""
    loads = [0.0] * cus
    for t in sorted(times, reverse=True):
        k = min(range(cus), key=lambda c: loads[c])
        loads[k] += t
    return max(loads) if times else 0.0


def contract_makespan(times: Sequence[float], cus: int = CUS) -> float:
    """A contraction's tiles: a last round that would fill at most half the
    CUs runs, after the full rounds, as a second launch of twice as many
    half-height tiles; the shortest tiles form that round."""
    n, r = len(times), len(times) % cus
    if n <= cus or r == 0 or 2 * r > cus:
        return makespan(times, cus)
    ts = sorted(times, reverse=True)
    half = [HALF_TILE * x for x in ts[n - r:] for _ in range(2)]
    return makespan(ts[:n - r], cus) + LAUNCH_US + makespan(half, cus)


def op_device_time(op: dict, counts: Dict[str, int]) -> float:
    """Microseconds of one operator's kernel under a spec: a contraction as
    256 x 256 output tiles per segment (output block), each doing its
    segment's whole contracted extent; attention as 128-query-row tiles, each
    seeing the keys of its segment's kept key blocks up to its last row; the
    memory-bound operators as their bytes at the copy rate."""
    numel_out = 1
    for c in op["out"]:
        numel_out *= op["ext"][c]
    if op["kind"] in ("rmsnorm", "swiglu", "add"):
        nbytes = 2 * (2 * numel_out + op["ext"][op["ins"][1][0]]) if op["kind"] == "rmsnorm" else 2 * 3 * numel_out
        return LAUNCH_US + nbytes / COPY_BPS * 1e6
    sp = {c: equal_splits(op["ext"][c], counts[c]) for c in op["letters"]}
    segs: Dict[tuple, list] = {}
    for cell in itertools.product(*[range(counts[c]) for c in op["letters"]]):
        at = dict(zip(op["letters"], cell))
        if op["causal"] is not None:
            s, t = op["causal"]
            if sp[t][at[t]] >= sp[s][at[s] + 1]:
                continue
        segs.setdefault(tuple(at[c] for c in op["out"]), []).append(at)
    size = lambda at, c: sp[c][at[c] + 1] - sp[c][at[c]]  # noqa: E731
    tiles: List[float] = []
    if op["kind"] == "contract":
        A, B_ = op["ins"]
        for cells in segs.values():
            nb = M = N = 1
            for c in op["out"]:
                if c in A and c in B_:
                    nb *= size(cells[0], c)
                elif c in A:
                    M *= size(cells[0], c)
                else:
                    N *= size(cells[0], c)
            K = 0
            for at in cells:
                k = 1
                for c in op["letters"]:
                    if c not in op["out"]:
                        k *= size(at, c)
                K += k
            n = nb * -(-M // 256) * -(-N // 256)
            tiles += [2.0 * 256 * 256 * K / GEMM_CU_FLOPS * 1e6] * n
    else:
        q, k = op["ins"][0], op["ins"][1]
        s, t, d = q[-2], k[-2], q[-1]
        for cells in segs.values():
            nbh = 1
            for c in q[:-2]:
                nbh *= size(cells[0], c)
            s_lo, S = sp[s][cells[0][s]], size(cells[0], s)
            for s0 in range(0, S, 128):
                last = s_lo + min(S, s0 + 128) - 1
                keys = 0
                for at in cells:
                    t_lo, t_hi = sp[t][at[t]], sp[t][at[t] + 1]
                    hi = min(t_hi, last + 1) if op["causal"] is not None else t_hi
                    keys += max(0, hi - t_lo)
                tiles += [4.0 * 128 * op["ext"][d] * keys / ATTN_CU_FLOPS * 1e6] * nbh
    return LAUNCH_US + (contract_makespan(tiles) if op["kind"] == "contract" else makespan(tiles))


def plan_device_time(g: Graph, plan: Sequence[Dict[str, int]]) -> float:
    """Every operator's modelled time, plus one copy launch per edge whose
    tilings differ or that leaves a view (each element read and written once,
    2 bytes each)."""
    total = 0.0
    for i, op in enumerate(g.ops):
        total += op_device_time(op, plan[i])
        for s, t in zip(op["ins"], op["inputs"]):
            q = g.producer[t]
            if t in g.view_of or (q is not None and tiling(s, plan[i]) != tiling(g.ops[q]["out"], plan[q])):
                total += LAUNCH_US + 2 * 2 * g.numel(t) / COPY_BPS * 1e6
    return total


def brute_force_device(g: Graph, p: int) -> float:
    """The least modelled time over every joint choice of specs."""
    return min(plan_device_time(g, plan) for plan in itertools.product(*[candidate_specs(op, p) for op in g.ops]))
