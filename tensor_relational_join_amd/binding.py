"""ctypes binding of libja's C ABI (include/ja.h).

Argument marshalling only: every function here forwards to the entry point of
the same name in libja.so, which runs the whole join-agg path in its HIP
kernels.  Device pointers and streams are plain integers (for example
``tensor.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``).
Failures raise JaError with the library's status and message.

If libja.so has not been built the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# JA_LIBJA names another build of the same library (the host-sanitizer build
# of `python -m tensor_relational_join_amd.build --sanitize`)
LIB_PATH = os.environ.get("JA_LIBJA") or os.path.join(_HERE, "libja.so")

JA_MAX_RANK = 8
JA_F32, JA_BF16, JA_F16 = 0, 1, 2
JA_AGG_SUM, JA_AGG_MAX, JA_AGG_SOFTMAX = 0, 1, 2
STATUS = {0: "JA_OK", -1: "JA_ERR_ARG", -2: "JA_ERR_SPEC", -3: "JA_ERR_DECOMP", -4: "JA_ERR_SHAPE",
          -5: "JA_ERR_DTYPE", -6: "JA_ERR_WORKSPACE", -7: "JA_ERR_UNSUPPORTED", -8: "JA_ERR_HIP",
          -9: "JA_ERR_STATE"}
DTYPE_SIZE = {JA_F32: 4, JA_BF16: 2, JA_F16: 2}


class JaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, "JA_ERR_UNKNOWN")
        super().__init__("%s: %s" % (self.name, message))


class ja_relation_desc(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * JA_MAX_RANK), ("nblk", ctypes.c_int32 * JA_MAX_RANK),
                ("splits", ctypes.POINTER(ctypes.c_int64) * JA_MAX_RANK)]


class ja_view(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("shape", ctypes.c_int64 * JA_MAX_RANK),
                ("perm", ctypes.c_int32 * JA_MAX_RANK)]


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_st = ctypes.c_int32
_descp = ctypes.POINTER(ja_relation_desc)
_descpp = ctypes.POINTER(_descp)
_viewp = ctypes.POINTER(ja_view)

# name -> (restype, argtypes)
_SIGS = {
    "ja_abi_version": (_i32, []),
    "ja_status_str": (ctypes.c_char_p, [_st]),
    "ja_last_error": (ctypes.c_char_p, []),
    "ja_relation_bytes": (_st, [_descp, ctypes.POINTER(_sz)]),
    "ja_relation_nblocks": (_st, [_descp, ctypes.POINTER(_i64)]),
    "ja_relation_block": (_st, [_descp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                ctypes.POINTER(_sz)]),
    "ja_spec_create": (_st, [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(_vp)]),
    "ja_spec_destroy": (None, [_vp]),
    "ja_spec_letters": (_st, [_vp, ctypes.c_char_p, _sz]),
    "ja_decomp_create": (_st, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i32),
                               ctypes.POINTER(ctypes.POINTER(_i64)), ctypes.POINTER(_vp)]),
    "ja_decomp_destroy": (None, [_vp]),
    "ja_join": (_st, [_vp, _vp, ctypes.POINTER(_vp)]),
    "ja_tuples_count": (_st, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "ja_tuples_export": (_st, [_vp, ctypes.POINTER(_i32), _i64, ctypes.POINTER(_i64), _i64]),
    "ja_tuples_destroy": (None, [_vp]),
    "ja_djoin_create": (_st, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i32), ctypes.POINTER(_vp)]),
    "ja_djoin_device_bytes": (_st, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_i64),
                                    ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ja_djoin_upload": (_st, [_vp, _vp, _sz, _vp]),
    "ja_djoin_run": (_st, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ja_djoin_destroy": (None, [_vp]),
    "ja_calibrate_mfma": (_st, [_i32, _i32, _vp, ctypes.POINTER(ctypes.c_double), _vp]),
    "ja_calibrate_copy": (_st, [_vp, _vp, _sz, _vp]),
    "ja_dattn_create": (_st, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i32), _i32, ctypes.POINTER(_vp)]),
    "ja_dattn_device_bytes": (_st, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_i64)]),
    "ja_dattn_upload": (_st, [_vp, _vp, _sz, _vp]),
    "ja_dattn_run": (_st, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ja_dattn_destroy": (None, [_vp]),
    "ja_graph_create": (_st, [ctypes.POINTER(_vp)]),
    "ja_graph_destroy": (None, [_vp]),
    "ja_graph_add_input": (_st, [_vp, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "ja_graph_add_op": (_st, [_vp, _vp, ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
    "ja_graph_add_view": (_st, [_vp, _i32, ctypes.POINTER(ja_view), _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "ja_graph_count": (_st, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "ja_graph_plan": (_st, [_vp, _i32, _i32, ctypes.c_uint64, ctypes.POINTER(ctypes.c_double)]),
    "ja_graph_plan_intervals": (_st, [_vp, _i32, ctypes.POINTER(_i32), _i32]),
    "ja_graph_cost": (_st, [_vp, ctypes.POINTER(ctypes.POINTER(_i32)), ctypes.POINTER(ctypes.c_double),
                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "ja_graph_device_time": (_st, [_vp, ctypes.POINTER(ctypes.POINTER(_i32)), ctypes.POINTER(ctypes.c_double)]),
    "ja_plan_create": (_st, [_vp, _vp, _descpp, _i32, _descp, ctypes.POINTER(_vp)]),
    "ja_plan_device_bytes": (_st, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "ja_plan_upload": (_st, [_vp, _vp, _sz, _vp]),
    "ja_plan_run": (_st, [_vp, ctypes.POINTER(_vp), _vp, _vp, _vp]),
    "ja_plan_partial_bytes": (_st, [_vp, ctypes.POINTER(_sz)]),
    "ja_kernel": (_st, [_vp, ctypes.POINTER(_vp), _vp, _vp]),
    "ja_agg": (_st, [_vp, _i32, _vp, _vp, _vp]),
    "ja_plan_destroy": (None, [_vp]),
    "ja_einsum_workspace_bytes": (_st, [_vp, _vp, _descpp, _i32, _descp, ctypes.POINTER(_sz)]),
    "ja_einsum": (_st, [_vp, _vp, _descpp, ctypes.POINTER(_vp), _i32, _descp, _vp, _vp, _sz, _vp]),
    "ja_einsum_noalloc": (_st, [_vp, _vp, _descpp, ctypes.POINTER(_vp), _i32, _descp, _vp, _vp]),
    "ja_repart_create": (_st, [_descp, _descp, _viewp, ctypes.POINTER(_vp)]),
    "ja_repart_count": (_st, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ja_repart_device_bytes": (_st, [_vp, ctypes.POINTER(_sz)]),
    "ja_repart_upload": (_st, [_vp, _vp, _sz, _vp]),
    "ja_repart_run": (_st, [_vp, _vp, _vp, _vp]),
    "ja_repart_destroy": (None, [_vp]),
    "ja_repartition_workspace_bytes": (_st, [_descp, _descp, _viewp, ctypes.POINTER(_sz)]),
    "ja_repartition": (_st, [_descp, _vp, _descp, _vp, _viewp, _vp, _sz, _vp]),
}

EXPORTED = sorted(_SIGS)

if not os.path.exists(LIB_PATH):
    raise ImportError("libja.so is not built (%s); run `python -m tensor_relational_join_amd.build`" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(st: int):
    if st != 0:
        raise JaError(st, _lib.ja_last_error().decode())


def raw():
    """The loaded ctypes library."""
    return _lib


# --------------------------------------------------------------------------- descriptors

class Relation:
    """Owner of a ja_relation_desc and its split arrays."""

    def __init__(self, shape: Sequence[int], nblk: Optional[Sequence[int]] = None,
                 splits: Optional[Sequence[Optional[Sequence[int]]]] = None, dtype: int = JA_BF16):
        rank = len(shape)
        if not 1 <= rank <= JA_MAX_RANK:
            raise ValueError("rank must be 1..8")
        self.shape = tuple(int(x) for x in shape)
        self.dtype = dtype
        d = ja_relation_desc()
        d.rank = rank
        d.dtype = dtype
        self._keep = []
        for i in range(rank):
            d.shape[i] = self.shape[i]
            sp = splits[i] if splits is not None else None
            if sp is not None:
                arr = (ctypes.c_int64 * len(sp))(*[int(x) for x in sp])
                self._keep.append(arr)
                d.splits[i] = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))
                d.nblk[i] = len(sp) - 1
            else:
                d.nblk[i] = int(nblk[i]) if nblk is not None else 1
        self.desc = d
        self.nblk = tuple(int(d.nblk[i]) for i in range(rank))
        # split points per dimension (near-equal reading where none were given)
        self.splits = []
        for i in range(rank):
            sp = splits[i] if splits is not None else None
            if sp is None:
                n, q = self.shape[i], self.nblk[i]
                base, extra = divmod(n, q)
                sp = [0]
                for j in range(q):
                    sp.append(sp[-1] + base + (1 if j < extra else 0))
            self.splits.append([int(x) for x in sp])

    @property
    def ptr(self):
        return ctypes.pointer(self.desc)

    @property
    def nbytes(self) -> int:
        # a relation is immutable once described: ask the library once
        if getattr(self, "_nbytes", None) is None:
            self._nbytes = ja_relation_bytes(self)
        return self._nbytes


def _desc_array(rels):
    arr = (_descp * len(rels))()
    for i, r in enumerate(rels):
        arr[i] = r.ptr
    return arr


def _ptr_array(ptrs):
    arr = (_vp * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = _vp(int(p))
    return arr


def make_view(shape: Sequence[int], perm: Sequence[int]) -> ja_view:
    v = ja_view()
    v.rank = len(shape)
    for i, (s, p) in enumerate(zip(shape, perm)):
        v.shape[i] = int(s)
        v.perm[i] = int(p)
    return v


# --------------------------------------------------------------------------- entry points

def ja_abi_version() -> int:
    return int(_lib.ja_abi_version())


def ja_status_str(status: int) -> str:
    return _lib.ja_status_str(status).decode()


def ja_last_error() -> str:
    return _lib.ja_last_error().decode()


def ja_relation_bytes(rel: Relation) -> int:
    n = _sz()
    _check(_lib.ja_relation_bytes(rel.ptr, ctypes.byref(n)))
    return n.value


def ja_relation_nblocks(rel: Relation) -> int:
    n = _i64()
    _check(_lib.ja_relation_nblocks(rel.ptr, ctypes.byref(n)))
    return n.value


def ja_relation_block(rel: Relation, key: Sequence[int]):
    r = len(rel.shape)
    k = (_i64 * r)(*key)
    lo, hi, off = (_i64 * r)(), (_i64 * r)(), _sz()
    _check(_lib.ja_relation_block(rel.ptr, k, lo, hi, ctypes.byref(off)))
    return tuple(lo), tuple(hi), off.value


def ja_spec_create(einsum: str, op: str, params: str = "") -> int:
    h = _vp()
    _check(_lib.ja_spec_create(einsum.encode(), op.encode(), params.encode(), ctypes.byref(h)))
    return h.value


def ja_spec_destroy(spec: int):
    _lib.ja_spec_destroy(_vp(spec))


def ja_spec_letters(spec: int) -> str:
    buf = ctypes.create_string_buffer(32)
    _check(_lib.ja_spec_letters(_vp(spec), buf, 32))
    return buf.value.decode()


def ja_decomp_create(spec: int, extents: Sequence[int], intervals: Sequence[int],
                     splits: Optional[Sequence[Optional[Sequence[int]]]] = None) -> int:
    n = len(extents)
    ext = (_i64 * n)(*extents)
    iv = (_i32 * n)(*intervals)
    sp = None
    keep = []
    if splits is not None:
        sp = (ctypes.POINTER(_i64) * n)()
        for i, s in enumerate(splits):
            if s is not None:
                arr = (_i64 * len(s))(*s)
                keep.append(arr)
                sp[i] = ctypes.cast(arr, ctypes.POINTER(_i64))
    h = _vp()
    _check(_lib.ja_decomp_create(_vp(spec), ext, iv, sp, ctypes.byref(h)))
    return h.value


def ja_decomp_destroy(decomp: int):
    _lib.ja_decomp_destroy(_vp(decomp))


def ja_join(spec: int, decomp: int) -> int:
    h = _vp()
    _check(_lib.ja_join(_vp(spec), _vp(decomp), ctypes.byref(h)))
    return h.value


def ja_tuples_count(tuples: int):
    nt, ns, nl = _i64(), _i64(), _i32()
    _check(_lib.ja_tuples_count(_vp(tuples), ctypes.byref(nt), ctypes.byref(ns), ctypes.byref(nl)))
    return nt.value, ns.value, nl.value


def ja_tuples_export(tuples: int):
    """(records as a list of per-letter interval indices, segment offsets)."""
    import numpy as np

    nt, ns, nl = ja_tuples_count(tuples)
    rec = np.zeros(max(nt * nl, 1), dtype=np.int32)
    seg = np.zeros(ns + 1, dtype=np.int64)
    _check(_lib.ja_tuples_export(_vp(tuples), rec.ctypes.data_as(ctypes.POINTER(_i32)), rec.size,
                                 seg.ctypes.data_as(ctypes.POINTER(_i64)), seg.size))
    return rec[: nt * nl].reshape(nt, nl), seg


def ja_tuples_destroy(tuples: int):
    _lib.ja_tuples_destroy(_vp(tuples))


def ja_djoin_create(spec: int, extents: Sequence[int], intervals: Sequence[int]) -> int:
    n = len(extents)
    h = _vp()
    _check(_lib.ja_djoin_create(_vp(spec), (_i64 * n)(*extents), (_i32 * n)(*intervals), ctypes.byref(h)))
    return h.value


def ja_djoin_device_bytes(join: int):
    """(table_bytes, workspace_bytes, max_tuples, max_segs, n_splits)."""
    tb, wb, mt, ms, ns = _sz(), _sz(), _i64(), _i64(), _i64()
    _check(_lib.ja_djoin_device_bytes(_vp(join), ctypes.byref(tb), ctypes.byref(wb), ctypes.byref(mt),
                                      ctypes.byref(ms), ctypes.byref(ns)))
    return tb.value, wb.value, mt.value, ms.value, ns.value


def ja_djoin_upload(join: int, dev_buf: int, nbytes: int, stream: int = 0):
    _check(_lib.ja_djoin_upload(_vp(join), _vp(dev_buf), nbytes, _vp(stream)))


def ja_djoin_run(join: int, splits_dev: int, rec: int, seg_off: int, counts: int, workspace: int, stream: int = 0):
    _check(_lib.ja_djoin_run(_vp(join), _vp(splits_dev), _vp(rec), _vp(seg_off), _vp(counts), _vp(workspace),
                             _vp(stream)))


def ja_djoin_destroy(join: int):
    _lib.ja_djoin_destroy(_vp(join))


def ja_calibrate_mfma(workgroups: int, iters: int, sink: int, stream: int = 0) -> float:
    """Enqueue the MFMA-loop ceiling kernel; returns the flops it performs."""
    f = ctypes.c_double()
    _check(_lib.ja_calibrate_mfma(workgroups, iters, _vp(sink), ctypes.byref(f), _vp(stream)))
    return f.value


def ja_calibrate_copy(src: int, dst: int, nbytes: int, stream: int = 0):
    _check(_lib.ja_calibrate_copy(_vp(src), _vp(dst), nbytes, _vp(stream)))


def ja_dattn_create(spec: int, extents: Sequence[int], intervals: Sequence[int], dtype: int = JA_BF16) -> int:
    n = len(extents)
    h = _vp()
    _check(_lib.ja_dattn_create(_vp(spec), (_i64 * n)(*extents), (_i32 * n)(*intervals), dtype, ctypes.byref(h)))
    return h.value


def ja_dattn_device_bytes(attn: int):
    """(table_bytes, workspace_bytes, n_splits)."""
    tb, wb, ns = _sz(), _sz(), _i64()
    _check(_lib.ja_dattn_device_bytes(_vp(attn), ctypes.byref(tb), ctypes.byref(wb), ctypes.byref(ns)))
    return tb.value, wb.value, ns.value


def ja_dattn_upload(attn: int, dev_buf: int, nbytes: int, stream: int = 0):
    _check(_lib.ja_dattn_upload(_vp(attn), _vp(dev_buf), nbytes, _vp(stream)))


def ja_dattn_run(attn: int, splits_dev: int, q: int, k: int, v: int, o: int, counts: int, workspace: int,
                 stream: int = 0):
    _check(_lib.ja_dattn_run(_vp(attn), _vp(splits_dev), _vp(q), _vp(k), _vp(v), _vp(o), _vp(counts),
                             _vp(workspace), _vp(stream)))


def ja_dattn_destroy(attn: int):
    _lib.ja_dattn_destroy(_vp(attn))


JA_PLAN_OPTIMAL, JA_PLAN_GREEDY, JA_PLAN_RANDOM, JA_PLAN_DEVICE = 0, 1, 2, 3


def ja_graph_create() -> int:
    h = _vp()
    _check(_lib.ja_graph_create(ctypes.byref(h)))
    return h.value


def ja_graph_destroy(graph: int):
    _lib.ja_graph_destroy(_vp(graph))


def ja_graph_add_input(graph: int, shape: Sequence[int]) -> int:
    t = _i32()
    _check(_lib.ja_graph_add_input(_vp(graph), len(shape), (_i64 * len(shape))(*shape), ctypes.byref(t)))
    return t.value


def ja_graph_add_op(graph: int, spec: int, inputs: Sequence[int]) -> int:
    t = _i32()
    _check(_lib.ja_graph_add_op(_vp(graph), _vp(spec), (_i32 * len(inputs))(*inputs), len(inputs), ctypes.byref(t)))
    return t.value


def ja_graph_add_view(graph: int, tensor: int, view: ja_view, shape: Sequence[int]) -> int:
    out = _i32()
    n = len(shape)
    _check(_lib.ja_graph_add_view(_vp(graph), tensor, ctypes.byref(view), n, (_i64 * n)(*shape), ctypes.byref(out)))
    return out.value


def ja_graph_count(graph: int):
    n_ops, n_t = _i32(), _i32()
    _check(_lib.ja_graph_count(_vp(graph), ctypes.byref(n_ops), ctypes.byref(n_t)))
    return n_ops.value, n_t.value


def ja_graph_plan(graph: int, p: int, mode: int = 0, seed: int = 0) -> float:
    c = ctypes.c_double()
    _check(_lib.ja_graph_plan(_vp(graph), p, mode, seed, ctypes.byref(c)))
    return c.value


def ja_graph_plan_intervals(graph: int, op: int, n_letters: int):
    buf = (_i32 * n_letters)()
    _check(_lib.ja_graph_plan_intervals(_vp(graph), op, buf, n_letters))
    return list(buf)


def ja_graph_cost(graph: int, intervals=None):
    """(repartition, join, aggregation) of the planned assignment, or of
    `intervals` (one list of interval counts per operator, letter order)."""
    r, j, a = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    arg = None
    if intervals is not None:
        rows = [(_i32 * len(v))(*v) for v in intervals]
        arg = (ctypes.POINTER(_i32) * len(rows))(*[ctypes.cast(x, ctypes.POINTER(_i32)) for x in rows])
    _check(_lib.ja_graph_cost(_vp(graph), arg, ctypes.byref(r), ctypes.byref(j), ctypes.byref(a)))
    return r.value, j.value, a.value


def ja_graph_device_time(graph: int, intervals=None) -> float:
    """The device-time model (microseconds) of the planned assignment, or of
    `intervals` (one list of interval counts per operator, letter order)."""
    us = ctypes.c_double()
    arg = None
    if intervals is not None:
        rows = [(_i32 * len(v))(*v) for v in intervals]
        arg = (ctypes.POINTER(_i32) * len(rows))(*[ctypes.cast(x, ctypes.POINTER(_i32)) for x in rows])
    _check(_lib.ja_graph_device_time(_vp(graph), arg, ctypes.byref(us)))
    return us.value


def ja_plan_create(spec: int, decomp: int, ins: Sequence[Relation], out: Relation) -> int:
    h = _vp()
    _check(_lib.ja_plan_create(_vp(spec), _vp(decomp), _desc_array(ins), len(ins), out.ptr, ctypes.byref(h)))
    return h.value


def ja_plan_device_bytes(plan: int):
    tb, wb = _sz(), _sz()
    _check(_lib.ja_plan_device_bytes(_vp(plan), ctypes.byref(tb), ctypes.byref(wb)))
    return tb.value, wb.value


def ja_plan_upload(plan: int, dev_buf: int, nbytes: int, stream: int = 0):
    _check(_lib.ja_plan_upload(_vp(plan), _vp(dev_buf), nbytes, _vp(stream)))


def ja_plan_run(plan: int, in_ptrs: Sequence[int], out_ptr: int, workspace: int = 0, stream: int = 0):
    _check(_lib.ja_plan_run(_vp(plan), _ptr_array(in_ptrs), _vp(out_ptr), _vp(workspace), _vp(stream)))


def ja_plan_partial_bytes(plan: int) -> int:
    n = _sz()
    _check(_lib.ja_plan_partial_bytes(_vp(plan), ctypes.byref(n)))
    return n.value


def ja_kernel(plan: int, in_ptrs: Sequence[int], partials: int, stream: int = 0):
    _check(_lib.ja_kernel(_vp(plan), _ptr_array(in_ptrs), _vp(partials), _vp(stream)))


def ja_agg(plan: int, op: int, partials: int, out_ptr: int, stream: int = 0):
    _check(_lib.ja_agg(_vp(plan), op, _vp(partials), _vp(out_ptr), _vp(stream)))


def ja_plan_destroy(plan: int):
    _lib.ja_plan_destroy(_vp(plan))


def ja_einsum_workspace_bytes(spec: int, decomp: int, ins: Sequence[Relation], out: Relation) -> int:
    n = _sz()
    _check(_lib.ja_einsum_workspace_bytes(_vp(spec), _vp(decomp), _desc_array(ins), len(ins), out.ptr,
                                          ctypes.byref(n)))
    return n.value


def ja_einsum(spec: int, decomp: int, ins: Sequence[Relation], in_ptrs: Sequence[int], out: Relation,
              out_ptr: int, dev_ws: int, ws_bytes: int, stream: int = 0):
    _check(_lib.ja_einsum(_vp(spec), _vp(decomp), _desc_array(ins), _ptr_array(in_ptrs), len(ins), out.ptr,
                          _vp(out_ptr), _vp(dev_ws), ws_bytes, _vp(stream)))


def ja_einsum_noalloc(spec: int, decomp: int, ins: Sequence[Relation], in_ptrs: Sequence[int], out: Relation,
                      out_ptr: int, stream: int = 0):
    _check(_lib.ja_einsum_noalloc(_vp(spec), _vp(decomp), _desc_array(ins), _ptr_array(in_ptrs), len(ins), out.ptr,
                                  _vp(out_ptr), _vp(stream)))


JA_NOALLOC_SCRATCH_BYTES = 32 << 20


def _view_ptr(view: Optional[ja_view]):
    return ctypes.pointer(view) if view is not None else None


def ja_repart_create(src: Relation, dst: Relation, view: Optional[ja_view] = None) -> int:
    h = _vp()
    _check(_lib.ja_repart_create(src.ptr, dst.ptr, _view_ptr(view), ctypes.byref(h)))
    return h.value


def ja_repart_count(rp: int):
    na, nt = _i64(), _i64()
    _check(_lib.ja_repart_count(_vp(rp), ctypes.byref(na), ctypes.byref(nt)))
    return na.value, nt.value


def ja_repart_device_bytes(rp: int) -> int:
    n = _sz()
    _check(_lib.ja_repart_device_bytes(_vp(rp), ctypes.byref(n)))
    return n.value


def ja_repart_upload(rp: int, dev_buf: int, nbytes: int, stream: int = 0):
    _check(_lib.ja_repart_upload(_vp(rp), _vp(dev_buf), nbytes, _vp(stream)))


def ja_repart_run(rp: int, src_ptr: int, dst_ptr: int, stream: int = 0):
    _check(_lib.ja_repart_run(_vp(rp), _vp(src_ptr), _vp(dst_ptr), _vp(stream)))


def ja_repart_destroy(rp: int):
    _lib.ja_repart_destroy(_vp(rp))


def ja_repartition_workspace_bytes(src: Relation, dst: Relation, view: Optional[ja_view] = None) -> int:
    n = _sz()
    _check(_lib.ja_repartition_workspace_bytes(src.ptr, dst.ptr, _view_ptr(view), ctypes.byref(n)))
    return n.value


def ja_repartition(src: Relation, src_ptr: int, dst: Relation, dst_ptr: int, view: Optional[ja_view],
                   dev_ws: int, ws_bytes: int, stream: int = 0):
    _check(_lib.ja_repartition(src.ptr, _vp(src_ptr), dst.ptr, _vp(dst_ptr), _view_ptr(view), _vp(dev_ws),
                               ws_bytes, _vp(stream)))
