"""CPU oracle for the join-agg hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library (neither imports
the other); the two meet only through the seeded input bytes.

What it computes, and where each piece comes from (the pages: "Every Kernel
Is a Join: Automatic Multi-GPU Parallelism for AI Computations in
Einsummable", paperpeel full text):

* dense results by their plain definitions, in float64 (``ja_oracle.c``):
  the loop-nest contraction, textbook two-pass attention, RMSNorm, SwiGLU,
  elementwise add;
* tensor types, projections and tilings (section 3.1, section 3.2);
* join-agg specs for an einsum, one function spec per combination of
  intervals of the shardable indices (section 3.3), executed by the
  three-phase definition Join / Aggregate / Recompose (section 3.2,
  Definition 3.7) -- ``execute_joinagg``;
* the degenerate relational join-agg in which every key is one cell and
  every value a scalar (section 1) -- ``brute_force_einsum``;
* canonical tuple lists with CSR segments -- ``tuple_records``;
* the overlay grid whose cells are the atoms of a repartition (section 5.3),
  and the repartition itself -- ``overlay_atoms``, ``repartition``;
* attention as a blocked join-agg with the online-softmax aggregation
  (m, l, acc) -- ``attention_online_blocked`` (the aggregation operator need
  not be addition, section 5.2), its per-tuple triples before aggregation
  and their fold -- ``attention_triples``, ``softmax_fold``; both attention forms take fewer key-value
  heads than query heads (grouped-query attention, section 3.3: query heads
  g*R .. g*R+R-1 share key-value head g), and ``attention`` /
  ``tuple_records`` take sequences packed end to end along the sequence index
  (section 3.3: attention never crosses a sequence boundary);
* a contraction followed by a 1:1 join on its output key, with nothing
  rounded in between (elementwise operators as joins, section 1) --
  ``contract_residual`` (A B + R) and ``contract_swiglu`` (silu(gate) * up
  over a (gate, up) pair letter);
* the LLaMA-shaped block as a chain of the above -- ``llama_block``, whose
  ``fused`` form leaves unrounded the contraction results that such a join
  consumes.

Readings where the pages are silent (listed again in the design notes):
intervals are half-open [lo, hi); near-equal intervals give the first
(n mod q) intervals one extra element; causal means key t is visible to query
s iff t <= s, and a (s-block, t-block) tuple is dropped when t_lo >= s_hi;
every materialised bf16 relation is rounded to nearest-even once, from the
exact (float64) value.
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libja_oracle.so")
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)


def build(force: bool = False) -> str:
    """Compile ja_oracle.c into libja_oracle.so with gcc -O3 + OpenMP (no
    -ffast-math, so every float64 operation keeps its order and rounding; no
    -march=native, since the library built here also runs on other hosts)."""
    import subprocess

    src = os.path.join(_HERE, "ja_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_bf16_to_f64.argtypes = [_u16p, ctypes.c_int64, _f64p]
        lib.orc_f64_to_bf16.argtypes = [_f64p, ctypes.c_int64, _u16p]
        lib.orc_f16_to_f64.argtypes = [_u16p, ctypes.c_int64, _f64p]
        lib.orc_f64_to_f16.argtypes = [_f64p, ctypes.c_int64, _u16p]
        lib.orc_einsum2.argtypes = [ctypes.c_char_p, _i64p, _f64p, _f64p, _f64p]
        lib.orc_einsum2.restype = ctypes.c_int
        lib.orc_einsum2_points.argtypes = [ctypes.c_char_p, _i64p, _f64p, _f64p, ctypes.c_int64, _i64p, _f64p]
        lib.orc_einsum2_points.restype = ctypes.c_int
        lib.orc_matmul.argtypes = [_f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        lib.orc_attention_rows.argtypes = [_f64p, _f64p, _f64p] + [ctypes.c_int64] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int64, _i64p, ctypes.c_int64, _i64p, _f64p]
        lib.orc_rmsnorm.argtypes = [_f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _f64p]
        lib.orc_swiglu.argtypes = [_f64p, _f64p, ctypes.c_int64, _f64p]
        lib.orc_add.argtypes = [_f64p, _f64p, ctypes.c_int64, _f64p]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------

def bf16_to_f64(h) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (uint16) to float64."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().orc_bf16_to_f64(_ptr(h, _u16p), h.size, _ptr(out, _f64p))
    return out


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns, nearest-even."""
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16(_ptr(x, _f64p), x.size, _ptr(out, _u16p))
    return out


def round_bf16(x) -> np.ndarray:
    """The float64 value of the bfloat16 nearest to x."""
    return bf16_to_f64(f64_to_bf16(x))


def f16_to_f64(h) -> np.ndarray:
    """Exact decode of IEEE half bit patterns (uint16) to float64."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().orc_f16_to_f64(_ptr(h, _u16p), h.size, _ptr(out, _f64p))
    return out


def f64_to_f16(x) -> np.ndarray:
    """Round float64 values to IEEE half bit patterns, nearest-even."""
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_f16(_ptr(x, _f64p), x.size, _ptr(out, _u16p))
    return out


def round_f16(x) -> np.ndarray:
    """The float64 value of the IEEE half nearest to x."""
    return f16_to_f64(f64_to_f16(x))


# --------------------------------------------------------------------------
# dense definitions
# --------------------------------------------------------------------------

def _parse(spec: str):
    lhs, out = spec.split("->")
    ins = lhs.split(",")
    return ins, out


def _ext26(spec: str, *ops) -> np.ndarray:
    ins, _ = _parse(spec)
    ext = np.zeros(26, dtype=np.int64)
    for s, a in zip(ins, ops):
        if len(s) != a.ndim:
            raise ValueError("operand rank does not match %r" % s)
        for c, n in zip(s, a.shape):
            l = ord(c) - ord("a")
            if ext[l] and ext[l] != n:
                raise ValueError("letter %s has two extents" % c)
            ext[l] = n
    return ext


def einsum(spec: str, A, B) -> np.ndarray:
    """Two-operand einsum by its definition: every output cell is the sum,
    over all values of the letters that do not reach the output, of the
    product of the two operand cells (float64 loop nest in C)."""
    A, B = _f64(A), _f64(B)
    ext = _ext26(spec, A, B)
    _, out = _parse(spec)
    shape = tuple(int(ext[ord(c) - 97]) for c in out)
    C = np.empty(shape, dtype=np.float64)
    rc = _load().orc_einsum2(spec.encode(), _ptr(ext, _i64p), _ptr(A, _f64p), _ptr(B, _f64p), _ptr(C, _f64p))
    if rc:
        raise ValueError("bad einsum spec %r" % spec)
    return C


def einsum_points(spec: str, A, B, points) -> np.ndarray:
    """The einsum evaluated only at the given output multi-indices
    (array [n, rank_out])."""
    A, B = _f64(A), _f64(B)
    ext = _ext26(spec, A, B)
    _, out = _parse(spec)
    shape = tuple(int(ext[ord(c) - 97]) for c in out)
    pts = np.asarray(points, dtype=np.int64).reshape(-1, len(out))
    lin = np.ascontiguousarray(np.ravel_multi_index(tuple(pts.T), shape).astype(np.int64))
    vals = np.empty(lin.size, dtype=np.float64)
    rc = _load().orc_einsum2_points(spec.encode(), _ptr(ext, _i64p), _ptr(A, _f64p), _ptr(B, _f64p),
                                    lin.size, _ptr(lin, _i64p), _ptr(vals, _f64p))
    if rc:
        raise ValueError("bad einsum spec %r" % spec)
    return vals


def matmul(A, B) -> np.ndarray:
    """C = A @ B for 2-D operands (float64, plain loops)."""
    A, B = _f64(A), _f64(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner extents differ")
    C = np.empty((M, N), dtype=np.float64)
    _load().orc_matmul(_ptr(A, _f64p), _ptr(B, _f64p), _ptr(C, _f64p), M, K, N)
    return C


def attention_rows(Q, K, V, rows, scale: float, causal: bool, seq_ends: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention output rows for the listed (b, h, s) query rows.
    Q [B,H,S,D], K/V [B,HK,T,D] with HK dividing H: query head h reads
    key-value head h // (H // HK) (grouped-query attention when HK < H,
    section 3.3; ordinary multi-head attention when HK = H).  With seq_ends
    (ascending, the last = S = T) the sequence index holds independent
    sequences packed end to end (section 3.3) and a key is visible to a query
    only inside the query's own sequence.  Two-pass softmax in float64."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Bn, H, S, D = Q.shape
    HK, T = K.shape[1], K.shape[2]
    if K.shape != V.shape or K.shape[0] != Bn or K.shape[3] != D or H % HK:
        raise ValueError("attention: K and V must be [B, HK, T, D] with HK dividing Q's H")
    ends = np.ascontiguousarray(np.asarray(seq_ends if seq_ends is not None else [], dtype=np.int64))
    if ends.size and (S != T or ends[-1] != S or np.any(np.diff(ends) <= 0) or ends[0] <= 0):
        raise ValueError("attention: sequence ends must ascend to S = T")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    _load().orc_attention_rows(_ptr(Q, _f64p), _ptr(K, _f64p), _ptr(V, _f64p), Bn, H, HK, S, T, D, float(scale),
                               1 if causal else 0, ends.size, _ptr(ends, _i64p) if ends.size else None,
                               rows.shape[0], _ptr(rows, _i64p), _ptr(out, _f64p))
    return out


def attention(Q, K, V, scale: float, causal: bool, seq_ends: Optional[Sequence[int]] = None) -> np.ndarray:
    Bn, H, S, D = np.shape(Q)
    rows = np.array(list(itertools.product(range(Bn), range(H), range(S))), dtype=np.int64)
    return attention_rows(Q, K, V, rows, scale, causal, seq_ends).reshape(Bn, H, S, D)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x, g = _f64(x), _f64(g)
    R, D = x.shape
    y = np.empty_like(x)
    _load().orc_rmsnorm(_ptr(x, _f64p), _ptr(g, _f64p), R, D, float(eps), _ptr(y, _f64p))
    return y


def swiglu(g, u) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    h = np.empty_like(g)
    _load().orc_swiglu(_ptr(g, _f64p), _ptr(u, _f64p), g.size, _ptr(h, _f64p))
    return h


def add(a, b) -> np.ndarray:
    a, b = _f64(a), _f64(b)
    c = np.empty_like(a)
    _load().orc_add(_ptr(a, _f64p), _ptr(b, _f64p), a.size, _ptr(c, _f64p))
    return c


def contract_residual(spec: str, A, B, R) -> np.ndarray:
    """A contraction followed by a 1:1 join with a residual relation on the
    output key (section 1: elementwise operators as joins): A B + R in
    float64, with no rounding in between.  spec: 'A,B->C'; R has C's shape."""
    return add(einsum(spec, A, B), R)


def contract_swiglu(spec: str, A, B) -> np.ndarray:
    """spec 'A,B->C' whose B ends with a letter (absent from A and C) of
    extent 2 that indexes a (gate, up) pair: the contraction into C's letters
    plus that letter, then the 1:1 join of the pair's members,
    silu(gate) * up, in float64 with no rounding in between."""
    lhs, out = spec.split("->")
    a, b = lhs.split(",")
    P = einsum("%s,%s->%s%s" % (a, b, out, b[-1]), A, B)
    return swiglu(P[..., 0], P[..., 1])


# --------------------------------------------------------------------------
# tensor types, tilings and relations (section 3.1, section 3.2)
# --------------------------------------------------------------------------

Box = Tuple[Tuple[int, ...], Tuple[int, ...]]  # (lower bounds, upper bounds), half-open


def equal_splits(n: int, q: int) -> List[int]:
    """Split points of [0, n) into q near-equal intervals; the first n mod q
    intervals are one longer."""
    if q < 1 or q > max(n, 1):
        raise ValueError("bad interval count")
    base, extra = divmod(n, q)
    pts = [0]
    for i in range(q):
        pts.append(pts[-1] + base + (1 if i < extra else 0))
    return pts


def box_cells(box: Box) -> int:
    lo, hi = box
    n = 1
    for a, b in zip(lo, hi):
        n *= max(0, b - a)
    return n


def tiles(boxes: Sequence[Box], shape: Sequence[int]) -> bool:
    """Section 3.1 tiling: the boxes cover the index set of the zero-bounded
    type `shape` and are pairwise disjoint (checked cell by cell)."""
    count = np.zeros(tuple(shape), dtype=np.int64)
    for lo, hi in boxes:
        if any(a < 0 or b > n or a > b for a, b, n in zip(lo, hi, shape)):
            return False
        count[tuple(slice(a, b) for a, b in zip(lo, hi))] += 1
    return bool(np.all(count == 1))


class Relation:
    """A tensor as a set of (key, block) pairs.  The key of a block is its
    coordinate in the per-dimension interval grid; the block is the
    projection of the tensor onto that box (section 3.2).  Stored layout
    (the oracle's own): blocks back to back in lexicographic key order (first
    dimension slowest), each block dense row-major over its box."""

    def __init__(self, shape: Sequence[int], splits: Sequence[Sequence[int]]):
        self.shape = tuple(int(n) for n in shape)
        self.splits = [list(map(int, s)) for s in splits]
        if len(self.splits) != len(self.shape):
            raise ValueError("one split list per dimension")
        for n, s in zip(self.shape, self.splits):
            if s[0] != 0 or s[-1] != n or any(b <= a for a, b in zip(s, s[1:])):
                raise ValueError("split points must rise strictly from 0 to the extent")

    @classmethod
    def even(cls, shape: Sequence[int], nblk: Sequence[int]) -> "Relation":
        return cls(shape, [equal_splits(n, q) for n, q in zip(shape, nblk)])

    @property
    def nblk(self) -> Tuple[int, ...]:
        return tuple(len(s) - 1 for s in self.splits)

    def keys(self):
        return itertools.product(*[range(q) for q in self.nblk])

    def box(self, key) -> Box:
        lo = tuple(self.splits[d][k] for d, k in enumerate(key))
        hi = tuple(self.splits[d][k + 1] for d, k in enumerate(key))
        return lo, hi

    def pack(self, dense: np.ndarray) -> np.ndarray:
        if tuple(dense.shape) != self.shape:
            raise ValueError("dense shape does not match the relation")
        parts = []
        for key in self.keys():
            lo, hi = self.box(key)
            parts.append(np.ascontiguousarray(dense[tuple(slice(a, b) for a, b in zip(lo, hi))]).ravel())
        return np.concatenate(parts) if parts else np.zeros(0, dtype=dense.dtype)

    def unpack(self, flat: np.ndarray) -> np.ndarray:
        dense = np.empty(self.shape, dtype=flat.dtype)
        off = 0
        for key in self.keys():
            lo, hi = self.box(key)
            n = box_cells((lo, hi))
            dense[tuple(slice(a, b) for a, b in zip(lo, hi))] = flat[off:off + n].reshape(
                tuple(b - a for a, b in zip(lo, hi)))
            off += n
        if off != flat.size:
            raise ValueError("flat buffer size does not match the relation")
        return dense


# --------------------------------------------------------------------------
# join-agg specs and their execution (section 3.2, section 3.3)
# --------------------------------------------------------------------------

class FunctionSpec:
    """One function specification: the projected input types and the
    projected output type, plus the interval index of every letter (the grid
    cell it came from)."""

    def __init__(self, cell: Dict[str, int], inputs: List[Box], output: Box):
        self.cell = cell
        self.inputs = inputs
        self.output = output


def letters_of(spec: str) -> List[str]:
    """Distinct letters in order of first appearance in the spec string."""
    out: List[str] = []
    for c in spec:
        if c.isalpha() and c not in out:
            out.append(c)
    return out


def joinagg_spec(spec: str, splits: Dict[str, Sequence[int]],
                 keep: Optional[Callable[[Dict[str, Tuple[int, int]]], bool]] = None) -> List[FunctionSpec]:
    """The join-agg spec an einsum-shaped operator returns for the given
    intervals of its shardable letters: one function specification per
    combination of intervals (section 3.3), each projecting every operand and
    the output onto the intervals of its letters.  `keep` is an optional join
    predicate over the intervals (used for dropping fully masked causal
    tuples)."""
    ins, out = _parse(spec)
    letters = letters_of(spec)
    ranges = [range(len(splits[c]) - 1) for c in letters]
    specs = []
    for combo in itertools.product(*ranges):
        cell = dict(zip(letters, combo))
        iv = {c: (splits[c][cell[c]], splits[c][cell[c] + 1]) for c in letters}
        if keep is not None and not keep(iv):
            continue
        in_boxes = [(tuple(iv[c][0] for c in s), tuple(iv[c][1] for c in s)) for s in ins]
        out_box = (tuple(iv[c][0] for c in out), tuple(iv[c][1] for c in out))
        specs.append(FunctionSpec(cell, in_boxes, out_box))
    return specs


def execute_joinagg(specs: List[FunctionSpec], inputs: Sequence[np.ndarray], out_shape: Sequence[int],
                    f: Callable[..., np.ndarray], oplus: Callable[[np.ndarray, np.ndarray], np.ndarray],
                    finalize: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> np.ndarray:
    """Definition 3.7 in three phases:
    (1) Join: project every input onto the spec's input types and run f;
    (2) Aggregate: combine with oplus, in ascending spec order, all outputs
        that share one output type;
    (3) Recompose: check the distinct output types tile the output, then
        stitch the aggregated blocks into the output tensor."""
    partials: Dict[Box, np.ndarray] = {}
    order: List[Box] = []
    for F in specs:  # (1) join
        blocks = [np.array(U[tuple(slice(a, b) for a, b in zip(*box))]) for U, box in zip(inputs, F.inputs)]
        part = f(*blocks)
        if F.output in partials:  # (2) aggregate
            partials[F.output] = oplus(partials[F.output], part)
        else:
            partials[F.output] = part
            order.append(F.output)
    if not tiles(order, out_shape):
        raise ValueError("output types do not tile the output (tiling condition violated)")
    out = None
    for box in order:  # (3) recompose
        blk = finalize(partials[box]) if finalize else partials[box]
        if out is None:
            out = np.zeros(tuple(out_shape), dtype=blk.dtype)
        out[tuple(slice(a, b) for a, b in zip(*box))] = blk
    return out


def contract_joinagg(spec: str, A, B, splits: Dict[str, Sequence[int]]) -> np.ndarray:
    """An einsum contraction executed as a join-agg: f is the block einsum,
    the aggregation is SUM (section 3.2, Examples 3.8 and 3.9)."""
    A, B = _f64(A), _f64(B)
    ins, out = _parse(spec)
    ext = {c: n for s, a in zip(ins, (A, B)) for c, n in zip(s, a.shape)}
    specs = joinagg_spec(spec, splits)
    return execute_joinagg(specs, [A, B], [ext[c] for c in out], lambda a, b: einsum(spec, a, b), np.add)


def brute_force_einsum(spec: str, A, B) -> np.ndarray:
    """The degenerate relational join-agg (section 1): each relation is a set
    of (cell index, scalar) pairs; natural join on the shared letters;
    multiply; group by the output letters; SUM.  Pure Python: tiny inputs."""
    ins, out = _parse(spec)
    A, B = np.asarray(A, dtype=np.float64), np.asarray(B, dtype=np.float64)
    relA = {idx: float(A[idx]) for idx in np.ndindex(A.shape)}
    relB = {idx: float(B[idx]) for idx in np.ndindex(B.shape)}
    shared = [c for c in ins[0] if c in ins[1]]
    # hash join: index B's tuples by the values of the shared letters
    table: Dict[tuple, list] = {}
    for idx, v in relB.items():
        key = tuple(idx[ins[1].index(c)] for c in shared)
        table.setdefault(key, []).append((idx, v))
    groups: Dict[tuple, float] = {}
    for ia, va in relA.items():
        key = tuple(ia[ins[0].index(c)] for c in shared)
        for ib, vb in table.get(key, []):
            val = {c: ia[ins[0].index(c)] for c in ins[0]}
            val.update({c: ib[ins[1].index(c)] for c in ins[1]})
            gk = tuple(val[c] for c in out)
            groups[gk] = groups.get(gk, 0.0) + va * vb
    ext = {c: n for s, a in zip(ins, (A, B)) for c, n in zip(s, a.shape)}
    C = np.zeros(tuple(ext[c] for c in out), dtype=np.float64)
    for k, v in groups.items():
        C[k] = v
    return C


def tuple_records(letters: Sequence[str], splits: Dict[str, Sequence[int]], group_by: Sequence[str],
                  causal: Optional[Tuple[str, str]] = None, packed: Optional[Tuple[str, str, Sequence[int]]] = None):
    """Canonical tuple list of a decomposition: one record per kept grid
    cell, holding the interval index of every letter (in `letters` order).
    Records are sorted by the group-by letters' indices (in `group_by`
    order), then by the other letters' indices (in `letters` order).  A
    causal pair (s, t) drops every cell whose key interval starts at or
    after the end of its query interval.  packed = (s, t, sequence ends)
    drops every cell whose query and key intervals share no sequence
    (section 3.3: attention never crosses a sequence boundary).  Returns
    (records [n, L] int32, segment offsets [nseg + 1] int64)."""
    rest = [c for c in letters if c not in group_by]
    recs = []
    for combo in itertools.product(*[range(len(splits[c]) - 1) for c in letters]):
        cell = dict(zip(letters, combo))
        if causal is not None:
            s, t = causal
            if splits[t][cell[t]] >= splits[s][cell[s] + 1]:
                continue
        if packed is not None:
            s, t, ends = packed
            slo, shi = splits[s][cell[s]], splits[s][cell[s] + 1]
            tlo, thi = splits[t][cell[t]], splits[t][cell[t] + 1]
            starts = [0] + list(ends[:-1])
            if not any(a < shi and b > slo and a < thi and b > tlo for a, b in zip(starts, ends)):
                continue
        recs.append(cell)
    recs.sort(key=lambda c: (tuple(c[x] for x in group_by), tuple(c[x] for x in rest)))
    arr = np.array([[c[x] for x in letters] for c in recs], dtype=np.int32).reshape(-1, len(letters))
    seg = [0]
    for i in range(1, len(recs)):
        if any(recs[i][x] != recs[i - 1][x] for x in group_by):
            seg.append(i)
    if recs:
        seg.append(len(recs))
    return arr, np.array(seg, dtype=np.int64)


# --------------------------------------------------------------------------
# attention as a blocked join-agg with the online-softmax aggregation
# --------------------------------------------------------------------------

def attention_online_blocked(Q, K, V, s_splits, t_splits, scale: float, causal: bool,
                             t_order: Optional[Callable[[List[int]], List[int]]] = None) -> np.ndarray:
    """Per (b, h, s-block) segment, each kept t-block tuple yields the
    triple (m, l, acc): m = row max of its scores, l = sum of exp(score - m),
    acc = sum of exp(score - m) * V.  Triples combine with
        m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
        acc = acc1 e^(m1-m) + acc2 e^(m2-m),
    which is associative and commutative with identity (-inf, 0, 0).  The
    output block is acc / l.  `t_order` may permute the fold order."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Bn, H, S, D = Q.shape
    rep = H // K.shape[1]  # query heads per key-value head (grouped-query attention when > 1)
    out = np.zeros_like(Q)
    for b in range(Bn):
        for h in range(H):
            kh = h // rep
            for si in range(len(s_splits) - 1):
                s0, s1 = s_splits[si], s_splits[si + 1]
                tis = [ti for ti in range(len(t_splits) - 1) if not (causal and t_splits[ti] >= s1)]
                if t_order is not None:
                    tis = t_order(tis)
                m = np.full(s1 - s0, -np.inf)
                l = np.zeros(s1 - s0)
                acc = np.zeros((s1 - s0, D))
                for ti in tis:
                    t0, t1 = t_splits[ti], t_splits[ti + 1]
                    sc = scale * (Q[b, h, s0:s1] @ K[b, kh, t0:t1].T)
                    if causal:
                        qs = np.arange(s0, s1)[:, None]
                        ks = np.arange(t0, t1)[None, :]
                        sc = np.where(ks <= qs, sc, -np.inf)
                    m2 = sc.max(axis=1)
                    p = np.where(np.isfinite(sc), np.exp(sc - np.where(np.isfinite(m2), m2, 0.0)[:, None]), 0.0)
                    l2 = p.sum(axis=1)
                    acc2 = p @ V[b, kh, t0:t1]
                    mn = np.maximum(m, m2)
                    a1 = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(mn), mn, 0.0)), 0.0)
                    a2 = np.where(np.isfinite(m2), np.exp(m2 - np.where(np.isfinite(mn), mn, 0.0)), 0.0)
                    l = l * a1 + l2 * a2
                    acc = acc * a1[:, None] + acc2 * a2[:, None]
                    m = mn
                out[b, h, s0:s1] = acc / l[:, None]
    return out


def attention_triples(Q, K, V, s_splits, t_splits, scale: float, causal: bool,
                      seq_ends: Optional[Sequence[int]] = None):
    """The per-tuple results of attention as a join-agg, before aggregation
    (section 3.2, Definition 3.7, step 1 -- f applied to every joined tuple):
    for every kept (b, h, s-block, t-block) tuple and each query row of the
    s-block, the triple over the keys of the t-block that the row may see
        m   = max of scale * q . k,
        l   = sum of exp(scale * q . k - m),
        acc = sum of exp(scale * q . k - m) * v
    (a row that sees none of the block's keys gets the identity (-inf, 0, 0)).
    Q [B,H,S,D], K/V [B,HK,T,D]; query head h reads key-value head
    h // (H // HK).  A tuple is kept unless causal drops it (its key block
    starts at or after the end of its query block) or, with seq_ends, its two
    blocks share no sequence.  Returns a list of ((b, h, si, ti), m, l, acc)
    in tuple order: grouped by (b, h, si), ti ascending."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Bn, H, S, D = Q.shape
    rep = H // K.shape[1]
    ends = list(seq_ends) if seq_ends is not None else None
    starts = [0] + ends[:-1] if ends else None

    def seq_id(pos):
        return np.searchsorted(np.asarray(ends), pos, side="right")

    out = []
    for b in range(Bn):
        for h in range(H):
            kh = h // rep
            for si in range(len(s_splits) - 1):
                s0, s1 = s_splits[si], s_splits[si + 1]
                for ti in range(len(t_splits) - 1):
                    t0, t1 = t_splits[ti], t_splits[ti + 1]
                    if causal and t0 >= s1:
                        continue
                    if ends and not any(a < s1 and e > s0 and a < t1 and e > t0 for a, e in zip(starts, ends)):
                        continue
                    sc = scale * (Q[b, h, s0:s1] @ K[b, kh, t0:t1].T)
                    qs = np.arange(s0, s1)[:, None]
                    ks = np.arange(t0, t1)[None, :]
                    vis = np.ones(sc.shape, dtype=bool)
                    if causal:
                        vis &= ks <= qs
                    if ends:
                        vis &= seq_id(ks) == seq_id(qs)
                    sc = np.where(vis, sc, -np.inf)
                    m = sc.max(axis=1)
                    mref = np.where(np.isfinite(m), m, 0.0)
                    p = np.where(vis, np.exp(sc - mref[:, None]), 0.0)
                    out.append(((b, h, si, ti), m, p.sum(axis=1), p @ V[b, kh, t0:t1]))
    return out


def softmax_fold(triples):
    """The aggregation of attention's per-tuple triples (section 5.2: the
    aggregation operator need not be addition): fold (m, l, acc) pairs with
        m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
        acc = acc1 e^(m1-m) + acc2 e^(m2-m),
    starting from the identity (-inf, 0, 0), in the order given.  Returns the
    folded (m, l, acc)."""
    m, l, acc = None, None, None
    for m2, l2, acc2 in triples:
        if m is None:
            m, l, acc = np.full_like(m2, -np.inf), np.zeros_like(l2), np.zeros_like(acc2)
        mn = np.maximum(m, m2)
        mref = np.where(np.isfinite(mn), mn, 0.0)
        a1 = np.where(np.isfinite(m), np.exp(m - mref), 0.0)
        a2 = np.where(np.isfinite(m2), np.exp(m2 - mref), 0.0)
        l = l * a1 + l2 * a2
        acc = acc * a1[:, None] + acc2 * a2[:, None]
        m = mn
    return m, l, acc


# --------------------------------------------------------------------------
# repartition (section 4.3 item 1, section 5.3)
# --------------------------------------------------------------------------

def apply_view(dense: np.ndarray, vshape: Optional[Sequence[int]], perm: Optional[Sequence[int]],
               out_shape: Sequence[int]) -> np.ndarray:
    """The logical re-indexing a repartition may apply: read the source
    row-major as `vshape`, permute axes (output axis k = view axis perm[k]),
    then read the result row-major as `out_shape`."""
    x = dense
    if vshape is not None:
        x = x.reshape(tuple(vshape))
    if perm is not None:
        x = np.transpose(x, tuple(perm))
    return np.ascontiguousarray(x).reshape(tuple(out_shape))


def repartition(src: Relation, src_flat: np.ndarray, dst: Relation, vshape=None, perm=None) -> np.ndarray:
    """Re-block a relation: the destination holds, block by block, exactly
    the elements of the (optionally re-indexed) source tensor."""
    dense = src.unpack(src_flat)
    return dst.pack(apply_view(dense, vshape, perm, dst.shape))


def overlay_atoms(*split_families: Sequence[Sequence[int]]) -> List[List[int]]:
    """Section 5.3 overlay: per dimension, the union of the lower and upper
    bounds of every block of every family.  The resulting grid's cells are
    the atoms; every block of every family is a disjoint union of atoms."""
    rank = len(split_families[0])
    return [sorted(set().union(*[set(fam[d]) for fam in split_families])) for d in range(rank)]


# --------------------------------------------------------------------------
# LLaMA-shaped block (pre-norm, causal MHA, SwiGLU FFN, two residual adds)
# --------------------------------------------------------------------------

def _qkv_heads(qkv, batch: int, seq: int, heads: int, kv_heads: int, hd: int):
    """Q [b, heads, s, hd], K and V [b, kv_heads, s, hd] from the fused
    projection's columns [Q heads | K heads | V heads], head h of each part in
    columns [h*hd, (h+1)*hd) of that part; token t = b*seq + s."""
    qd, kd = heads * hd, kv_heads * hd
    Q = qkv[:, :qd].reshape(batch, seq, heads, hd).transpose(0, 2, 1, 3)
    K = qkv[:, qd:qd + kd].reshape(batch, seq, kv_heads, hd).transpose(0, 2, 1, 3)
    V = qkv[:, qd + kd:qd + 2 * kd].reshape(batch, seq, kv_heads, hd).transpose(0, 2, 1, 3)
    return Q, K, V


def _rounder(dtype: str):
    """The rounding of a materialised relation: bf16 or IEEE half, nearest even."""
    if dtype == "bf16":
        return round_bf16
    if dtype == "f16":
        return round_f16
    raise ValueError("dtype is 'bf16' or 'f16'")


def llama_block(x, g1, w_qkv, w_o, g2, w_gate, w_up, w_down, batch: int, seq: int, heads: int,
                eps: float = 1e-6, return_intermediates: bool = False, kv_heads: Optional[int] = None,
                fused: bool = False, dtype: str = "bf16"):
    """Float64 reference of one transformer block on bf16 inputs, with every
    materialised relation rounded to bf16.  x [batch*seq, d]; w_qkv is
    [d, (heads + 2 kv_heads) hd] = [W_q | W_k | W_v] with head h in columns
    [h*hd, (h+1)*hd) of each part; kv_heads < heads is grouped-query
    attention (query head h reads key-value head h // (heads // kv_heads),
    section 3.3), kv_heads = heads (the default) multi-head attention.
    Token t = b*seq + s.  No rotary embedding and no biases.

    fused: the block whose residual adds and SwiGLU are 1:1 joins applied
    inside the producing contractions, so the output projection, the gate
    and up projections and the down projection are never materialised and
    are not rounded; every relation that is written still is.

    dtype: the format every materialised relation is rounded to, "bf16" or
    "f16" (IEEE half; the pages run their blocks in FP16, section 6.1)."""
    T, Dm = x.shape
    hd = Dm // heads
    kv_heads = heads if kv_heads is None else kv_heads
    r = _rounder(dtype)
    rc = (lambda v: v) if fused else r  # contraction outputs consumed by a 1:1 join
    h1 = r(rmsnorm(x, g1, eps))
    qkv = r(matmul(h1, w_qkv))
    Q, K, V = _qkv_heads(qkv, batch, seq, heads, kv_heads, hd)
    O = r(attention(Q, K, V, 1.0 / np.sqrt(hd), True))
    o = O.transpose(0, 2, 1, 3).reshape(T, Dm)
    a = rc(matmul(o, w_o))
    x2 = r(add(x, a))
    h2 = r(rmsnorm(x2, g2, eps))
    gt = rc(matmul(h2, w_gate))
    up = rc(matmul(h2, w_up))
    f = r(swiglu(gt, up))
    d = rc(matmul(f, w_down))
    y = r(add(x2, d))
    if return_intermediates:
        return y, dict(h1=h1, qkv=qkv, O=O, a=a, x2=x2, h2=h2, gate=gt, up=up, f=f, d=d)
    return y


def llama_block_tokens(x, g1, w_qkv, w_o, g2, w_gate, w_up, w_down, batch: int, seq: int, heads: int,
                       tokens, eps: float = 1e-6, kv_heads: Optional[int] = None, fused: bool = False,
                       dtype: str = "bf16"):
    """The same block as `llama_block`, evaluated only at the listed tokens
    (t = b*seq + s).  Keys and values are formed for every position up to the
    largest listed s of each batch, as causal attention needs them.  Every
    row is computed exactly as in the full version, so the rows agree with
    it bit for bit."""
    x = _f64(x)
    T, Dm = x.shape
    hd = Dm // heads
    kv_heads = heads if kv_heads is None else kv_heads
    r = _rounder(dtype)
    rc = (lambda v: v) if fused else r
    tokens = np.asarray(tokens, dtype=np.int64)
    y = np.empty((tokens.size, Dm))
    for b in sorted(set((tokens // seq).tolist())):
        sel = np.nonzero(tokens // seq == b)[0]
        ss = tokens[sel] % seq
        smax = int(ss.max())
        rows = x[b * seq: b * seq + smax + 1]
        h1 = r(rmsnorm(rows, g1, eps))
        qkv = r(matmul(h1, w_qkv))
        Q, K, V = _qkv_heads(qkv, 1, smax + 1, heads, kv_heads, hd)
        q_rows = np.array([(0, h, s) for s in ss for h in range(heads)], dtype=np.int64)
        O = r(attention_rows(Q, K, V, q_rows, 1.0 / np.sqrt(hd), True)).reshape(len(ss), heads * hd)
        a = rc(matmul(O, w_o))
        x2 = r(add(rows[ss], a))
        h2 = r(rmsnorm(x2, g2, eps))
        f = r(swiglu(rc(matmul(h2, w_gate)), rc(matmul(h2, w_up))))
        y[sel] = r(add(x2, rc(matmul(f, w_down))))
    return y
