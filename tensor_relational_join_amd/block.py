"""A LLaMA-shaped transformer block as a graph of join-agg operators.

Pre-norm block, causal multi-head attention, SwiGLU feed-forward, two
residual adds, no rotary embedding and no biases:

    h1 = rmsnorm(x, g1)               rd,d->rd      r: 2  d: 2
    qkv = h1 @ W_qkv                  td,dn->tn     t: 2  d: 2  n: 2   (3-D matmul decomposition, 8 tuples)
    Q, K, V = heads(qkv)              repartition [t, 3*dm] -> [3, b, h, s, hd], blocks [1,1,1,128,128]
    O = attention(Q, K, V)            bhsd,bhtd,bhtd->bhsd   b, h unit intervals, s and t 128-blocks, causal
    o = tokens(O)                     repartition [b, h, s, hd] -> [t, dm], blocks [t/2, dm/2]
    a = o @ W_o                       tm,mn->tn     t: 2  m: 2  n: 2
    x2 = x + a                        1:1 join on [t/2, dm/2] blocks
    h2 = rmsnorm(x2, g2)
    gt = h2 @ W_gate, up = h2 @ W_up  td,df->tf     t: 2  d: 2  f: 4
    f = silu(gt) * up                 1:1 join on [t/2, ffn/4] blocks
    dn = f @ W_down                   tf,fn->tn     t: 2  f: 4  n: 2
    y = x2 + dn

Only the QKV decomposition is fixed by the workload; the others are chosen
so that every producer's output blocking is its consumer's input blocking
(the repartition sub-cost of the pages' cost model, section 4.3, is then
zero for them), which leaves exactly the two re-indexing repartitions around
attention (tokens <-> heads).  That is the layout="heads" form above.

The default, layout="tokens", needs no repartition at all: attention's
relations keep the projections' token-major layout, the heads inside a row
(a block (b, s-interval) is 128 whole token rows of every head):

    h1 = rmsnorm(x, g1)               rd,d->rd      r: 1  d: 2
    qkv = h1 @ W_qkv                  td,dn->tn     t: 1  d: 2  n: cut at the Q | K | V column boundaries
    O = attention(Q, K, V)            bshd,bthd,bthd->bshd   b unit intervals, s and t 128-blocks, h whole
                                      (bsgrd,btgd,btgd->bsgrd with grouped key-value heads)
    a = O @ W_o                       tm,mn->tn     t: 1  m: 1  n: 2
    (every other op as above, with the tokens in one block)

The projection's Q, K and V column blocks are three contiguous [t, *]
arrays, exactly the relations Q [b, s, h, d], K and V [b, t, h, d] blocked
by (b, 128-interval of s or t), and attention's output O [b, s, h, d] is the
output projection's A [t, dm] as one block.

With kv_heads < heads the block uses grouped-query attention (the pages'
section 3.3: query heads g*R .. g*R+R-1 read key-value head g, R = heads /
kv_heads), the shape of the pages' own LLaMA-3-8B-like blocks:

    qkv = h1 @ W_qkv                  td,dn->tn     t: 1  d: 2  n: cut at the Q | K | V column boundaries
    (every other op as above, with the tokens in one block)
    Q = q_heads(qkv[Q part])          repartition [t, heads*hd] -> [b, g, r, s, hd], blocks [1,1,R,128,128]
    K, V = kv_heads(qkv[K, V parts])  repartition [t, kv*hd] -> [b, g, s, hd], blocks [1,1,128,128]
    O = attention(Q, K, V)            bgrsd,bgtd,bgtd->bgrsd   b, g unit intervals, s and t 128-blocks
    o = tokens(O)                     repartition [b, g, r, s, hd] -> [t, dm]

With t unsplit, the three column blocks of the projection's output are
three contiguous [t, *] arrays, each re-blocked on its own.

Every relation is bf16, or IEEE half with dtype=JA_F16 (the pages run
their blocks in FP16, section 6.1); the contractions accumulate in fp32.

With fused=True the two residual adds and SwiGLU are 1:1 joins applied by
the producing contractions to each aggregated block before it is written,
and the gate and up projections are one contraction whose weight pairs the
two matrices column by column (W_gu[d, f, 0] = W_gate[d, f], W_gu[d, f, 1] =
W_up[d, f]):

    x2 = o @ W_o + x                  tm,mn,tn->tn  contract_add     t: 2  m: 2  n: 2
    f = swiglu(h2 @ W_gu)             td,dfc->tf    contract_swiglu  t: 2  d: 2  f: 4  c: whole
    y = f @ W_down + x2               tf,fn,tn->tn  contract_add     t: 2  f: 4  n: 2

The projections a, gt, up and dn are then never written (nor rounded).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import binding as B
from .device import Op as _Op
from .device import Repart, alloc, equal_splits

# the steps in execution order (head-major layout), and the contractions among them
STEPS = ["norm1", "qkv", "to_heads", "attn", "to_tokens", "oproj", "add1", "norm2", "gate", "up", "swiglu",
         "down", "add2"]
GEMMS = ["qkv", "oproj", "gate", "up", "down"]
FUSED_STEPS = ["norm1", "qkv", "to_heads", "attn", "to_tokens", "oproj_add", "norm2", "gate_up", "down_add"]
FUSED_GEMMS = ["qkv", "oproj_add", "gate_up", "down_add"]
LAYOUTS = ("tokens", "heads")
SPLIT_TILES = 128


def _out_tiles(op) -> int:
    """256 x 256 output tiles of a contraction over its output blocks."""
    lhs, out = op.einsum.split("->")
    n = 1
    for c in out[-2:]:
        sp = op.splits[c]
        n *= sum(-(-(hi - lo) // 256) for lo, hi in zip(sp[:-1], sp[1:]))
    for c in out[:-2]:
        n *= op.splits[c][-1] - op.splits[c][0]
    return n


def _k_tuples(op) -> int:
    """Tuples per segment: the intervals of the contracted letters."""
    lhs, out = op.einsum.split("->")
    n = 1
    for c in set(lhs.replace(",", "")) - set(out):
        n *= len(op.splits[c]) - 1
    return n


class LlamaBlock:
    def __init__(self, batch: int = 4, seq: int = 2048, dm: int = 4096, heads: int = 32, ffn: int = 11008,
                 eps: float = 1e-6, device="cuda", kv_heads: Optional[int] = None, fused: bool = False,
                 dtype: int = B.JA_BF16, layout: str = "tokens", split_small: bool = True):
        if dm % heads or dm // heads != 128 or seq % 128:
            raise ValueError("the attention kernel needs head_dim 128 and 128-multiples of seq")
        if dtype not in (B.JA_BF16, B.JA_F16):
            raise ValueError("the block's relations are bf16 or IEEE half")
        if layout not in LAYOUTS:
            raise ValueError("layout is 'tokens' (attention on the projections' token-major relations) or 'heads'")
        self.dtype, self.layout = dtype, layout
        tok = layout == "tokens"
        kv = heads if kv_heads is None else kv_heads
        if kv <= 0 or heads % kv:
            raise ValueError("kv_heads must divide heads")
        self.batch, self.seq, self.dm, self.heads, self.ffn, self.eps = batch, seq, dm, heads, ffn, eps
        self.kv_heads, self.gqa, self.fused = kv, kv != heads, fused
        self.steps, self.gemms = (FUSED_STEPS, FUSED_GEMMS) if fused else (STEPS, GEMMS)
        if tok:
            self.steps = [n for n in self.steps if n not in ("to_heads", "to_tokens")]
        self.hd = dm // heads
        T = batch * seq
        self.T = T
        kvd = kv * self.hd
        self.qkv_cols = dm + 2 * kvd
        # tokens in two blocks; one block with grouped key-value heads, where the
        # projection's output must keep its Q, K, V parts contiguous
        t2, d2 = (equal_splits(T, 2) if not (self.gqa or tok) else [0, T]), equal_splits(dm, 2)
        f4 = equal_splits(ffn, 4)
        ep = "eps=%r" % eps
        nb = seq // 128
        self.ops: Dict[str, Op] = {}

        def Op(einsum, op, splits, params="", device="cuda", in_splits=None):  # noqa: N802 -- the block's dtype
            n_in = len(einsum.split("->")[0].split(","))
            return _Op(einsum, op, splits, params, [dtype] * n_in, dtype, device=device, in_splits=in_splits)

        self.ops["norm1"] = Op("rd,d->rd", "rmsnorm", {"r": t2, "d": d2}, ep, device=device)
        if tok:
            # the projection's Q, K, V parts are three contiguous token-major
            # arrays, which are attention's relations as they are: a block
            # (b, s-interval) holds whole rows of every head
            self.ops["qkv"] = Op("td,dn->tn", "contract",
                                 {"t": t2, "d": d2, "n": [0, dm, dm + kvd, dm + 2 * kvd]}, device=device)
            bs = {"b": equal_splits(batch, batch), "s": equal_splits(seq, nb), "t": equal_splits(seq, nb),
                  "d": [0, self.hd]}
            if not self.gqa:
                self.ops["attn"] = Op("bshd,bthd,bthd->bshd", "attention", {**bs, "h": [0, heads]}, "causal=s,t",
                                      device=device)
            else:
                self.ops["attn"] = Op("bsgrd,btgd,btgd->bsgrd", "attention",
                                      {**bs, "g": [0, kv], "r": [0, heads // kv]}, "causal=s,t", device=device)
        elif not self.gqa:
            self.ops["qkv"] = Op("td,dn->tn", "contract", {"t": t2, "d": d2, "n": equal_splits(3 * dm, 2)},
                                 device=device)
            att_sp = {"b": equal_splits(batch, batch), "h": equal_splits(heads, heads), "s": equal_splits(seq, nb),
                      "t": equal_splits(seq, nb), "d": [0, self.hd]}
            self.ops["attn"] = Op("bhsd,bhtd,bhtd->bhsd", "attention", att_sp, "causal=s,t", device=device)
        else:
            self.ops["qkv"] = Op("td,dn->tn", "contract",
                                 {"t": t2, "d": d2, "n": [0, dm, dm + kvd, dm + 2 * kvd]}, device=device)
            att_sp = {"b": equal_splits(batch, batch), "g": equal_splits(kv, kv), "r": [0, heads // kv],
                      "s": equal_splits(seq, nb), "t": equal_splits(seq, nb), "d": [0, self.hd]}
            self.ops["attn"] = Op("bgrsd,bgtd,bgtd->bgrsd", "attention", att_sp, "causal=s,t", device=device)
        # attention's token-major output is the projection's A as it is (m whole)
        m2 = [0, dm] if tok else d2
        # With few output tiles the projection's m is cut in four anyway (so
        # that it can run split into K tuples, below) while its A stays one
        # block: each tuple reads a sub-box of attention's token-major output.
        self._o_in = None
        if tok and split_small and -(-T // 256) * sum(-(-(b - a) // 256) for a, b in zip(d2[:-1], d2[1:])) \
                <= SPLIT_TILES:
            m2, self._o_in = equal_splits(dm, 4), [{"m": [0, dm]}]
        if not fused:
            self.ops["oproj"] = Op("tm,mn->tn", "contract", {"t": t2, "m": m2, "n": d2}, device=device,
                                   in_splits=self._o_in)
            self.ops["add1"] = Op("td,td->td", "add", {"t": t2, "d": d2}, device=device)
        else:
            self.ops["oproj_add"] = Op("tm,mn,tn->tn", "contract_add", {"t": t2, "m": m2, "n": d2}, device=device,
                                       in_splits=self._o_in)
        self.ops["norm2"] = Op("rd,d->rd", "rmsnorm", {"r": t2, "d": d2}, ep, device=device)
        if not fused:
            self.ops["gate"] = Op("td,df->tf", "contract", {"t": t2, "d": d2, "f": f4}, device=device)
            self.ops["up"] = Op("td,df->tf", "contract", {"t": t2, "d": d2, "f": f4}, device=device)
            self.ops["swiglu"] = Op("tf,tf->tf", "swiglu", {"t": t2, "f": f4}, device=device)
            self.ops["down"] = Op("tf,fn->tn", "contract", {"t": t2, "f": f4, "n": d2}, device=device)
            self.ops["add2"] = Op("td,td->td", "add", {"t": t2, "d": d2}, device=device)
        else:
            self.ops["gate_up"] = Op("td,dfc->tf", "contract_swiglu", {"t": t2, "d": d2, "f": f4, "c": [0, 2]},
                                     device=device)
            self.ops["down_add"] = Op("tf,fn,tn->tn", "contract_add", {"t": t2, "f": f4, "n": d2}, device=device)
        oproj = self.ops["oproj_add" if fused else "oproj"]
        # token-major <-> head-major re-blockings around attention
        self.rp: Dict[str, Repart] = {}
        if tok:
            pass
        elif not self.gqa:
            heads_rel = B.Relation((3, batch, heads, seq, self.hd), nblk=(3, batch, heads, nb, 1), dtype=dtype)
            self.rp["to_heads"] = Repart(self.ops["qkv"].out_rel, heads_rel,
                                         B.make_view((batch, seq, 3, heads, self.hd), (2, 0, 3, 1, 4)),
                                         device=device)
            self.rp["to_tokens"] = Repart(self.ops["attn"].out_rel, oproj.in_rels[0],
                                          B.make_view((batch, heads, seq, self.hd), (0, 2, 1, 3)), device=device)
            self.heads_rel = heads_rel
        else:
            rep = heads // kv
            q_rel, k_rel, v_rel = self.ops["attn"].in_rels
            self.part_rel = {"q": B.Relation((T, dm), nblk=(1, 1), dtype=dtype),
                             "k": B.Relation((T, kvd), nblk=(1, 1), dtype=dtype),
                             "v": B.Relation((T, kvd), nblk=(1, 1), dtype=dtype)}
            self.rp["to_q"] = Repart(self.part_rel["q"], q_rel,
                                     B.make_view((batch, seq, kv, rep, self.hd), (0, 2, 3, 1, 4)), device=device)
            for name, rel in (("k", k_rel), ("v", v_rel)):
                self.rp["to_" + name] = Repart(self.part_rel[name], rel,
                                               B.make_view((batch, seq, kv, self.hd), (0, 2, 1, 3)), device=device)
            self.rp["to_tokens"] = Repart(self.ops["attn"].out_rel, oproj.in_rels[0],
                                          B.make_view((batch, kv, rep, seq, self.hd), (0, 3, 1, 2, 4)),
                                          device=device)
        # relations of the block's inputs (materialised straight into the blockings the ops need)
        self.x_rel = self.ops["norm1"].in_rels[0]
        self.g_rel = self.ops["norm1"].in_rels[1]
        o = self.ops
        if not fused:
            self.w_rel = {"w_qkv": o["qkv"].in_rels[1], "w_o": o["oproj"].in_rels[1], "w_gate": o["gate"].in_rels[1],
                          "w_up": o["up"].in_rels[1], "w_down": o["down"].in_rels[1]}
        else:
            # w_gu [d, f, 2]: gate and up weights paired column by column
            self.w_rel = {"w_qkv": o["qkv"].in_rels[1], "w_o": o["oproj_add"].in_rels[1],
                          "w_gu": o["gate_up"].in_rels[1], "w_down": o["down_add"].in_rels[1]}
        # the block's output relation
        self.y_rel = o["down_add" if fused else "add2"].out_rel
        # intermediates
        if tok:
            heads = {}
        elif not self.gqa:
            heads = {"heads": alloc(self.heads_rel, device)}
        else:
            heads = {n: alloc(r, device) for n, r in zip("qkv", o["attn"].in_rels)}
        self.buf = {
            "h1": alloc(o["norm1"].out_rel, device), "qkv": alloc(o["qkv"].out_rel, device),
            **heads, "O": alloc(o["attn"].out_rel, device),
            "x2": alloc(oproj.out_rel, device), "h2": alloc(o["norm2"].out_rel, device),
        }
        # the projection's input: attention's output itself in the token-major layout
        self.buf["o"] = self.buf["O"] if tok else alloc(oproj.in_rels[0], device)
        if not fused:
            self.buf.update({"a": alloc(o["oproj"].out_rel, device), "gt": alloc(o["gate"].out_rel, device),
                             "up": alloc(o["up"].out_rel, device), "f": alloc(o["swiglu"].out_rel, device),
                             "dn": alloc(o["down"].out_rel, device)})
        else:
            self.buf["f"] = alloc(o["gate_up"].out_rel, device)
        # Contractions with few output tiles (at most SPLIT_TILES 256 x 256
        # tiles, under half of the 256 compute units) and at least two tuples
        # per segment run unfused: every tuple's partial block in parallel
        # (ja_kernel), then the atomic-free SUM of each segment's partials in
        # tuple order (ja_agg), so that the K tuples occupy compute units the
        # output tiles alone would leave idle.  A residual add fused into such
        # a contraction becomes a 1:1 join of its own after the SUM.
        self.split: Dict[str, str] = {}
        if split_small:
            for name in ("qkv", "oproj", "oproj_add", "down", "down_add"):
                op = self.ops.get(name)
                if op is not None and _out_tiles(op) <= SPLIT_TILES and _k_tuples(op) >= 2:
                    self.split[name] = name
        if "down_add" in self.split:
            sp = self.ops["down_add"].splits
            self.ops["down_split"] = Op("tf,fn->tn", "contract", {c: sp[c] for c in "tfn"}, device=device)
            self.ops["add2_split"] = Op("td,td->td", "add", {"t": sp["t"], "d": sp["n"]}, device=device)
            self.split["down_add"] = "down_split"
            self.buf["dn"] = alloc(self.ops["down_split"].out_rel, device)
        if "oproj_add" in self.split:
            sp = self.ops["oproj_add"].splits
            self.ops["oproj_split"] = Op("tm,mn->tn", "contract", {c: sp[c] for c in "tmn"}, device=device,
                                         in_splits=self._o_in)
            self.ops["add1_split"] = Op("td,td->td", "add", {"t": sp["t"], "d": sp["n"]}, device=device)
            self.split["oproj_add"] = "oproj_split"
            self.buf["a"] = alloc(self.ops["oproj_split"].out_rel, device)
        if self.split:
            self.partials = torch.empty(max(self.ops[v].partial_bytes() for v in self.split.values()) // 4,
                                        dtype=torch.float32, device=device)

    # ---------------------------------------------------------------- flops / bytes
    def flops(self) -> Dict[str, float]:
        T, dm, ffn = self.T, self.dm, self.ffn
        f = {"qkv": 2.0 * T * dm * self.qkv_cols, "oproj": 2.0 * T * dm * dm, "gate": 2.0 * T * dm * ffn,
             "up": 2.0 * T * dm * ffn, "down": 2.0 * T * ffn * dm}
        nb = self.seq // 128
        kept = nb * (nb + 1) // 2  # kept (s-block, t-block) tuples per (b, h)
        f["attn"] = 2 * 2.0 * 128 * 128 * self.hd * kept * self.batch * self.heads
        if self.fused:
            f["oproj_add"] = f.pop("oproj")
            f["gate_up"] = f.pop("gate") + f.pop("up")
            f["down_add"] = f.pop("down")
        return f

    def step_bytes(self) -> Dict[str, float]:
        """Algorithmic HBM bytes of the memory-bound steps (inputs read once,
        outputs written once)."""
        T, dm, ffn = self.T, self.dm, self.ffn
        e = 2.0
        b = {"norm1": e * (2 * T * dm + dm), "norm2": e * (2 * T * dm + dm)}
        if self.layout == "heads":
            b.update({"to_heads": e * 2 * T * self.qkv_cols, "to_tokens": e * 2 * T * dm})
        if not self.fused:
            b.update({"add1": e * 3 * T * dm, "add2": e * 3 * T * dm, "swiglu": e * 3 * T * ffn})
        return b

    # ---------------------------------------------------------------- execution
    def forward(self, x: torch.Tensor, w: Dict[str, torch.Tensor], y: torch.Tensor,
                events: Optional[Dict[str, List]] = None, stream=None):
        """One pass of the block.  x, y and the weights are device buffers in
        the relations' layouts (x_rel, w_rel, g_rel).  If `events` is given,
        a (start, end) torch event pair is recorded around every step."""
        o, b = self.ops, self.buf
        tok = self.layout == "tokens"
        if tok:
            nq, nk = self.T * self.dm, self.T * self.kv_heads * self.hd
            q, k, v = b["qkv"][:nq], b["qkv"][nq:nq + nk], b["qkv"][nq + nk:]
            to_heads = None
        elif not self.gqa:
            n = self.T * self.heads * self.hd  # elements of each of Q, K, V
            q, k, v = b["heads"][:n], b["heads"][n:2 * n], b["heads"][2 * n:]

            def to_heads():
                self.rp["to_heads"].run(b["qkv"], b["heads"], stream)
        else:
            q, k, v = b["q"], b["k"], b["v"]
            nq, nk = self.T * self.dm, self.T * self.kv_heads * self.hd  # the projection's Q and K, V parts

            def to_heads():
                self.rp["to_q"].run(b["qkv"][:nq], q, stream)
                self.rp["to_k"].run(b["qkv"][nq:nq + nk], k, stream)
                self.rp["to_v"].run(b["qkv"][nq + nk:], v, stream)
        def contract(name, ins, out):
            """op `name`, fused, or split into per-tuple partials and their SUM
            (the residual, if any, added after it as a 1:1 join)"""
            if name not in self.split:
                o[name].run(ins, out, stream)
                return
            sop = o[self.split[name]]
            sop.kernel(ins[:2], self.partials, stream)
            if name == "down_add":
                sop.agg(self.partials, b["dn"], stream=stream)
                o["add2_split"].run([ins[2], b["dn"]], out, stream)
            elif name == "oproj_add":
                sop.agg(self.partials, b["a"], stream=stream)
                o["add1_split"].run([ins[2], b["a"]], out, stream)
            else:
                sop.agg(self.partials, out, stream=stream)

        plan = [
            ("norm1", lambda: o["norm1"].run([x, w["g1"]], b["h1"], stream)),
            ("qkv", lambda: contract("qkv", [b["h1"], w["w_qkv"]], b["qkv"])),
            ("to_heads", to_heads),
            ("attn", lambda: o["attn"].run([q, k, v], b["O"], stream)),
            ("to_tokens", lambda: self.rp["to_tokens"].run(b["O"], b["o"], stream)),
        ]
        if tok:
            plan = [st for st in plan if st[0] not in ("to_heads", "to_tokens")]
        if not self.fused:
            plan += [
                ("oproj", lambda: contract("oproj", [b["o"], w["w_o"]], b["a"])),
                ("add1", lambda: o["add1"].run([x, b["a"]], b["x2"], stream)),
                ("norm2", lambda: o["norm2"].run([b["x2"], w["g2"]], b["h2"], stream)),
                ("gate", lambda: o["gate"].run([b["h2"], w["w_gate"]], b["gt"], stream)),
                ("up", lambda: o["up"].run([b["h2"], w["w_up"]], b["up"], stream)),
                ("swiglu", lambda: o["swiglu"].run([b["gt"], b["up"]], b["f"], stream)),
                ("down", lambda: contract("down", [b["f"], w["w_down"]], b["dn"])),
                ("add2", lambda: o["add2"].run([b["x2"], b["dn"]], y, stream)),
            ]
        else:
            plan += [
                ("oproj_add", lambda: contract("oproj_add", [b["o"], w["w_o"], x], b["x2"])),
                ("norm2", lambda: o["norm2"].run([b["x2"], w["g2"]], b["h2"], stream)),
                ("gate_up", lambda: o["gate_up"].run([b["h2"], w["w_gu"]], b["f"], stream)),
                ("down_add", lambda: contract("down_add", [b["f"], w["w_down"], b["x2"]], y)),
            ]
        for name, fn in plan:
            if events is not None:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                fn()
                e.record()
                events.setdefault(name, []).append((s, e))
            else:
                fn()

    # ---------------------------------------------------------------- inputs
    def materialize(self, dense: torch.Tensor, rel: B.Relation) -> torch.Tensor:
        """Copy a dense row-major device tensor (the block's dtype) into `rel`'s blocking
        with ja_repartition (a dense tensor is the relation with one block)."""
        src = B.Relation(rel.shape, nblk=[1] * len(rel.shape), dtype=rel.dtype)
        out = alloc(rel, dense.device)
        rp = Repart(src, rel, device=dense.device)
        try:
            rp.run(dense.reshape(-1), out)
        finally:
            torch.cuda.synchronize()
            rp.close()
        return out

    def dense(self, t: torch.Tensor, rel: B.Relation) -> torch.Tensor:
        """The inverse of `materialize`: a relation back to a dense tensor."""
        dst = B.Relation(rel.shape, nblk=[1] * len(rel.shape), dtype=rel.dtype)
        out = alloc(dst, t.device)
        rp = Repart(rel, dst, device=t.device)
        try:
            rp.run(t, out)
        finally:
            torch.cuda.synchronize()
            rp.close()
        return out.reshape(rel.shape)

    def close(self):
        for op in self.ops.values():
            op.close()
        for rp in self.rp.values():
            rp.close()
