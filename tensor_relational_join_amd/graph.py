"""Computation graphs: planned by the logical optimizer of libja
(ja_graph_*: "Every Kernel Is a Join", section 4) and run on one GPU with
libja's operators and repartitions.

``Graph`` records computation inputs and abstract operators (an einsum, an
op kind, params, input tensor ids) and asks ja_graph_plan for one join-agg
spec per operator: interval counts per letter, cut into near-equal
intervals.  ``PlannedRun`` runs one such plan: every operator with its
spec's decomposition; a computation input is materialised directly in the
blocking its consumer asks for (section 4.3: no repartition is charged for
it); an operator output whose blocking differs from what its consumer asks
for goes through a repartition (ja_repart_*), exactly the edges the proxy
charges.  Every step runs in libja's kernels on torch's current stream.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import binding as B
from .device import Op, Repart, alloc, equal_splits


class Graph:
    def __init__(self):
        self.shapes: List[Tuple[int, ...]] = []
        self.producer: List[Optional[int]] = []
        self.ops: List[dict] = []  # einsum, kind, params, inputs, letters
        self.views: Dict[int, Tuple[int, Tuple[int, ...], Tuple[int, ...]]] = {}  # tensor -> (source, vshape, perm)

    def input(self, shape: Sequence[int]) -> int:
        self.shapes.append(tuple(int(x) for x in shape))
        self.producer.append(None)
        return len(self.shapes) - 1

    def view(self, t: int, vshape: Sequence[int], perm: Sequence[int], shape: Sequence[int]) -> int:
        """Tensor t read row-major as vshape, its axes permuted (axis k of the
        result is axis perm[k]), read row-major as `shape` (ja_graph_add_view;
        realised by a repartition through the view)."""
        self.shapes.append(tuple(int(x) for x in shape))
        self.producer.append(None)
        self.views[len(self.shapes) - 1] = (t, tuple(vshape), tuple(perm))
        return len(self.shapes) - 1

    def op(self, einsum: str, kind: str, inputs: Sequence[int], params: str = "") -> int:
        lhs, out = einsum.split("->")
        ext: Dict[str, int] = {}
        for s, t in zip(lhs.split(","), inputs):
            if len(s) != len(self.shapes[t]):
                raise ValueError("input rank does not match the einsum")
            for c, e in zip(s, self.shapes[t]):
                if ext.setdefault(c, e) != e:
                    raise ValueError("letter %s has two extents" % c)
        spec = B.ja_spec_create(einsum, kind, params)
        letters = B.ja_spec_letters(spec)
        B.ja_spec_destroy(spec)
        self.ops.append(dict(einsum=einsum, kind=kind, params=params, inputs=list(inputs), letters=letters,
                             ext=ext, ins=lhs.split(","), out=out))
        self.shapes.append(tuple(ext[c] for c in out))
        self.producer.append(len(self.ops) - 1)
        return len(self.shapes) - 1

    def _lib(self):
        g = B.ja_graph_create()
        try:
            ids = {}
            for t, shape in enumerate(self.shapes):
                if t in self.views:
                    src, vshape, perm = self.views[t]
                    ids[t] = B.ja_graph_add_view(g, ids[src], B.make_view(vshape, perm), list(shape))
                elif self.producer[t] is None:
                    ids[t] = B.ja_graph_add_input(g, list(shape))
                else:
                    op = self.ops[self.producer[t]]
                    spec = B.ja_spec_create(op["einsum"], op["kind"], op["params"])
                    try:
                        ids[t] = B.ja_graph_add_op(g, spec, [ids[x] for x in op["inputs"]])
                    finally:
                        B.ja_spec_destroy(spec)
            return g
        except Exception:
            B.ja_graph_destroy(g)
            raise

    def plan(self, p: int, mode: int = B.JA_PLAN_OPTIMAL, seed: int = 0) -> Tuple[float, List[Dict[str, int]]]:
        """(proxy cost, interval counts per operator) chosen by ja_graph_plan."""
        g = self._lib()
        try:
            cost = B.ja_graph_plan(g, p, mode, seed)
            plan = [dict(zip(op["letters"], B.ja_graph_plan_intervals(g, i, len(op["letters"]))))
                    for i, op in enumerate(self.ops)]
            return cost, plan
        finally:
            B.ja_graph_destroy(g)

    def cost(self, plan: Sequence[Dict[str, int]]) -> Tuple[float, float, float]:
        """(repartition, join, aggregation) of the proxy for a plan."""
        g = self._lib()
        try:
            return B.ja_graph_cost(g, [[spec[c] for c in op["letters"]] for spec, op in zip(plan, self.ops)])
        finally:
            B.ja_graph_destroy(g)

    def device_time(self, plan: Sequence[Dict[str, int]]) -> float:
        """The device-time model of a plan, in microseconds."""
        g = self._lib()
        try:
            return B.ja_graph_device_time(g, [[spec[c] for c in op["letters"]] for spec, op in zip(plan, self.ops)])
        finally:
            B.ja_graph_destroy(g)


class PlannedRun:
    """One plan of a Graph, built on the current device (bf16 relations)."""

    def __init__(self, graph: Graph, plan: Sequence[Dict[str, int]], device="cuda", splits=None):
        """splits: per operator, explicit split points per letter instead of
        the plan's near-equal intervals (a hand-chosen decomposition)."""
        self.g = graph
        self.ops: List[Op] = []
        # (op, slot, repart, buffer): the repartition feeding an input slot, from its
        # producer's output (through the view when the slot reads a view)
        self.reparts: List[Tuple[int, int, Repart, torch.Tensor]] = []
        self.rep_src: Dict[Tuple[int, int], int] = {}  # (op, slot) -> the operator whose output it re-blocks
        self.input_slots: List[Tuple[int, int]] = []  # (op, slot) fed by a computation input (maybe through a view)
        self.outs: List[torch.Tensor] = []
        self.in_bufs: Dict[Tuple[int, int], torch.Tensor] = {}
        try:
            for i, op in enumerate(graph.ops):
                sp = splits[i] if splits is not None else {c: equal_splits(op["ext"][c], plan[i][c])
                                                            for c in op["letters"]}
                o = Op(op["einsum"], op["kind"], sp, op["params"], device=device)
                self.ops.append(o)
                self.outs.append(alloc(o.out_rel, device))
            for i, op in enumerate(graph.ops):
                for k, t in enumerate(op["inputs"]):
                    src, view = t, None
                    if t in graph.views:
                        src, vshape, perm = graph.views[t]
                        view = B.make_view(vshape, perm)
                    q = graph.producer[src]
                    want = self.ops[i].in_rels[k]
                    if q is None:
                        self.input_slots.append((i, k))
                        self.in_bufs[(i, k)] = alloc(want, device)
                    elif view is not None or self.ops[q].out_rel.splits != want.splits:
                        buf = alloc(want, device)
                        self.reparts.append((i, k, Repart(self.ops[q].out_rel, want, view, device=device), buf))
                        self.rep_src[(i, k)] = q
                        self.in_bufs[(i, k)] = buf
                    else:
                        self.in_bufs[(i, k)] = self.outs[q]
        except Exception:
            self.close()
            raise

    def load(self, dense: Dict[int, torch.Tensor]):
        """Materialise every computation input (dense row-major bf16 device
        tensors by tensor id) in the blocking each consumer asks for, through
        libja's repartition from a one-block relation."""
        for (i, k) in self.input_slots:
            t = self.g.ops[i]["inputs"][k]
            view = None
            if t in self.g.views:
                t, vshape, perm = self.g.views[t]
                view = B.make_view(vshape, perm)
            want = self.ops[i].in_rels[k]
            src = B.Relation(self.g.shapes[t], dtype=want.dtype)
            rp = Repart(src, want, view)
            try:
                rp.run(dense[t].contiguous().view(-1), self.in_bufs[(i, k)])
            finally:
                rp.close()

    def run(self):
        """Every operator in order, each after the repartitions of its inputs."""
        by_op: Dict[int, list] = {}
        for (i, k, rp, buf) in self.reparts:
            by_op.setdefault(i, []).append((k, rp, buf))
        for i, op in enumerate(self.g.ops):
            for (k, rp, buf) in by_op.get(i, []):
                rp.run(self.outs[self.rep_src[(i, k)]], buf)
            self.ops[i].run([self.in_bufs[(i, k)] for k in range(len(op["inputs"]))], self.outs[i])

    def dense_output(self, i: int) -> torch.Tensor:
        """Operator i's output as a dense row-major tensor."""
        rel = self.ops[i].out_rel
        dst = B.Relation(rel.shape)
        out = alloc(dst, self.outs[i].device)
        rp = Repart(rel, dst)
        try:
            rp.run(self.outs[i], out)
        finally:
            rp.close()
        return out.view(rel.shape)

    def close(self):
        for o in self.ops:
            o.close()
        for (_, _, rp, _) in self.reparts:
            rp.close()
        self.ops, self.reparts = [], []


def llama_block_graph(batch: int, seq: int, dm: int, heads: int, ffn: int, eps: float = 1e-6):
    """The LLaMA-shaped block (pre-norm, causal multi-head attention, SwiGLU
    feed-forward, two residual adds, no rotary embedding, no biases) as a
    graph of the pages' operators for the logical optimizer: the Q, K and V
    projections as three contractions, views between the token-major
    projections and the head-major attention, and every add and SwiGLU an
    operator of its own.  Returns (graph, tensor ids by name)."""
    T, hd = batch * seq, dm // heads
    g = Graph()
    t = {n: g.input(sh) for n, sh in (("x", (T, dm)), ("g1", (dm,)), ("w_q", (dm, dm)), ("w_k", (dm, dm)),
                                      ("w_v", (dm, dm)), ("w_o", (dm, dm)), ("g2", (dm,)), ("w_gate", (dm, ffn)),
                                      ("w_up", (dm, ffn)), ("w_down", (ffn, dm)))}
    ep = "eps=%r" % eps
    t["h1"] = g.op("rd,d->rd", "rmsnorm", [t["x"], t["g1"]], ep)
    heads_view = ((batch, seq, heads, hd), (0, 2, 1, 3), (batch, heads, seq, hd))
    for n in "qkv":
        t[n] = g.op("td,dn->tn", "contract", [t["h1"], t["w_" + n]])
        t[n.upper()] = g.view(t[n], *heads_view)
    t["O"] = g.op("bhsd,bhtd,bhtd->bhsd", "attention", [t["Q"], t["K"], t["V"]], "causal=s,t")
    t["o"] = g.view(t["O"], (batch, heads, seq, hd), (0, 2, 1, 3), (T, dm))
    t["a"] = g.op("tm,mn->tn", "contract", [t["o"], t["w_o"]])
    t["x2"] = g.op("td,td->td", "add", [t["x"], t["a"]])
    t["h2"] = g.op("rd,d->rd", "rmsnorm", [t["x2"], t["g2"]], ep)
    t["gt"] = g.op("td,df->tf", "contract", [t["h2"], t["w_gate"]])
    t["up"] = g.op("td,df->tf", "contract", [t["h2"], t["w_up"]])
    t["f"] = g.op("tf,tf->tf", "swiglu", [t["gt"], t["up"]])
    t["dn"] = g.op("tf,fn->tn", "contract", [t["f"], t["w_down"]])
    t["y"] = g.op("td,td->td", "add", [t["x2"], t["dn"]])
    return g, t


def llama_block_hand_splits(g: Graph, batch: int, seq: int) -> List[Dict[str, List[int]]]:
    """The hand-chosen decompositions of the LlamaBlock class (unfused), on
    the graph of llama_block_graph: tokens in two blocks and the model
    dimension in two everywhere, the FFN dimension in four, projections 2 x 2
    x 2, attention per (batch, head) with 128-blocks on both sequence
    indices."""
    out = []
    for op in g.ops:
        ext = op["ext"]
        sp = {}
        for c in op["letters"]:
            n = ext[c]
            if op["kind"] == "attention":
                q = {"b": batch, "h": ext["h"], "s": seq // 128, "t": seq // 128, "d": 1}[c]
            else:
                q = 4 if c == "f" else 2  # the FFN letter of the gate, up, SwiGLU and down operators
            sp[c] = equal_splits(n, q)
        out.append(sp)
    return out
