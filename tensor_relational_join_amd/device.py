"""Device-side conveniences over the C ABI: torch provides device memory and
streams; every computation goes through libja's entry points.

* ``Op``      -- an operator with a decomposition and its uploaded plan
                 (ja_spec_create / ja_decomp_create / ja_plan_create /
                 ja_plan_upload / ja_plan_run).
* ``Repart``  -- an uploaded repartition plan (ja_repart_*).
* ``alloc``   -- a device buffer for a relation.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import binding as B
from .binding import JA_BF16, JA_F16, JA_F32, Relation  # noqa: F401

TORCH_DTYPE = {JA_F32: torch.float32, JA_BF16: torch.bfloat16, JA_F16: torch.float16}


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def alloc(rel: Relation, device="cuda") -> torch.Tensor:
    """A flat device buffer holding one relation (torch allocations are
    256-byte aligned)."""
    n = rel.nbytes // B.DTYPE_SIZE[rel.dtype]
    return torch.empty(n, dtype=TORCH_DTYPE[rel.dtype], device=device)


def _check_layout(t, nbytes: int, dtype: Optional[torch.dtype], what: str):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s: expected a torch tensor, got %s" % (what, type(t).__name__))
    if not t.is_contiguous():
        raise ValueError("%s: the tensor must be contiguous" % what)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (what, t.dtype, dtype))
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s: %d bytes, the relation needs %d" % (what, have, nbytes))


def check_buffers(bufs):
    """Device addresses of the (tensor, nbytes, dtype, name) entries of
    `bufs` after checking that a kernel may read or write `nbytes` bytes of
    elements of `dtype` (None: any) in each: a contiguous tensor of that
    dtype, at least that large, on a GPU.  The library checks only pointer
    alignment, so a short or mistyped buffer would otherwise be read or
    written out of bounds on the device.  Every buffer's layout is checked
    before any buffer's device.  Raises ValueError."""
    for t, n, dt, what in bufs:
        _check_layout(t, n, dt, what)
    for t, _, _, what in bufs:
        if not t.is_cuda:
            raise ValueError("%s: the tensor must be on the GPU (device %s)" % (what, t.device))
    return [t.data_ptr() for t, _, _, _ in bufs]


def check_buffer(t, nbytes: int, dtype: Optional[torch.dtype], what: str) -> int:
    """check_buffers for one buffer."""
    return check_buffers([(t, nbytes, dtype, what)])[0]


def _rel_bufs(ts: Sequence[torch.Tensor], rels: Sequence[Relation], what: str):
    if len(ts) != len(rels):
        raise ValueError("%s: %d tensors for %d relations" % (what, len(ts), len(rels)))
    return [(t, r.nbytes, TORCH_DTYPE[r.dtype], "%s %d" % (what, i)) for i, (t, r) in enumerate(zip(ts, rels))]


def _table(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(16, (nbytes + 15) // 16 * 16), dtype=torch.uint8, device=device)


def relation_for(letters: str, splits: Dict[str, Sequence[int]], dtype: int) -> Relation:
    """The relation blocked exactly as the decomposition cuts its letters."""
    return Relation([splits[c][-1] for c in letters], splits=[list(splits[c]) for c in letters], dtype=dtype)


def equal_splits(n: int, q: int):
    base, extra = divmod(n, q)
    pts = [0]
    for i in range(q):
        pts.append(pts[-1] + base + (1 if i < extra else 0))
    return pts


class Op:
    """One operator, one decomposition, one plan uploaded to the device.

    einsum/op/params as in ja_spec_create; `splits` maps every letter to its
    interval boundaries (0 ... extent).  Relations default to the blocking
    the decomposition asks for; dtypes default to bf16."""

    def __init__(self, einsum: str, op: str, splits: Dict[str, Sequence[int]], params: str = "",
                 in_dtypes: Optional[Sequence[int]] = None, out_dtype: int = JA_BF16, device="cuda",
                 stream: Optional[torch.cuda.Stream] = None,
                 in_splits: Optional[Sequence[Optional[Dict[str, Sequence[int]]]]] = None):
        """in_splits: per input, an optional blocking of its own letters (a
        contraction operand of two letters may be blocked coarser than the
        decomposition; its tuples then read sub-boxes of its blocks)."""
        self.einsum, self.op = einsum, op
        self.splits = {c: list(v) for c, v in splits.items()}
        self.spec = B.ja_spec_create(einsum, op, params)
        self.decomp = None
        self.plan = None
        try:
            self.letters = B.ja_spec_letters(self.spec)
            ext = [splits[c][-1] for c in self.letters]
            iv = [len(splits[c]) - 1 for c in self.letters]
            self.decomp = B.ja_decomp_create(self.spec, ext, iv, [list(splits[c]) for c in self.letters])
            lhs, out = einsum.split("->")
            ins = lhs.split(",")
            in_dtypes = in_dtypes or [JA_BF16] * len(ins)
            in_splits = list(in_splits or []) + [None] * len(ins)
            self.in_rels = [relation_for(s, {**splits, **(own or {})}, dt)
                            for s, dt, own in zip(ins, in_dtypes, in_splits)]
            self.out_rel = relation_for(out, splits, out_dtype)
            self.plan = B.ja_plan_create(self.spec, self.decomp, self.in_rels, self.out_rel)
            tb, wb = B.ja_plan_device_bytes(self.plan)
            self.table = _table(tb, device)
            self.workspace = _table(wb, device) if wb else None
            B.ja_plan_upload(self.plan, self.table.data_ptr(), self.table.numel(), stream_handle(stream))
        except Exception:
            self.close()
            raise

    def tuples(self):
        t = B.ja_join(self.spec, self.decomp)
        try:
            return B.ja_tuples_export(t)
        finally:
            B.ja_tuples_destroy(t)

    def run(self, ins: Sequence[torch.Tensor], out: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
        ptrs = check_buffers(_rel_bufs(ins, self.in_rels, "input") +
                             [(out, self.out_rel.nbytes, TORCH_DTYPE[self.out_rel.dtype], "output")])
        ws = self.workspace.data_ptr() if self.workspace is not None else 0
        B.ja_plan_run(self.plan, ptrs[:-1], ptrs[-1], ws, stream_handle(stream))

    def partial_bytes(self) -> int:
        return B.ja_plan_partial_bytes(self.plan)

    def partial_buffer(self) -> torch.Tensor:
        return torch.empty(self.partial_bytes() // 4, dtype=torch.float32, device=self.table.device)

    def kernel(self, ins: Sequence[torch.Tensor], partials: torch.Tensor, stream=None):
        ptrs = check_buffers(_rel_bufs(ins, self.in_rels, "input") +
                             [(partials, self.partial_bytes(), torch.float32, "partials")])
        B.ja_kernel(self.plan, ptrs[:-1], ptrs[-1], stream_handle(stream))

    def agg(self, partials: torch.Tensor, out: torch.Tensor, op: int = B.JA_AGG_SUM, stream=None):
        pptr, optr = check_buffers([(partials, self.partial_bytes(), torch.float32, "partials"),
                                    (out, self.out_rel.nbytes, TORCH_DTYPE[self.out_rel.dtype], "output")])
        B.ja_agg(self.plan, op, pptr, optr, stream_handle(stream))

    def close(self):
        if self.plan:
            B.ja_plan_destroy(self.plan)
            self.plan = None
        if self.decomp:
            B.ja_decomp_destroy(self.decomp)
            self.decomp = None
        if self.spec:
            B.ja_spec_destroy(self.spec)
            self.spec = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Repart:
    """An uploaded re-blocking plan from `src` to `dst` (optional view)."""

    def __init__(self, src: Relation, dst: Relation, view: Optional[B.ja_view] = None, device="cuda",
                 stream: Optional[torch.cuda.Stream] = None):
        self.src, self.dst, self.view = src, dst, view
        self.rp = B.ja_repart_create(src, dst, view)
        try:
            self.n_atoms, self.n_tasks = B.ja_repart_count(self.rp)
            self.table = _table(B.ja_repart_device_bytes(self.rp), device)
            B.ja_repart_upload(self.rp, self.table.data_ptr(), self.table.numel(), stream_handle(stream))
        except Exception:
            self.close()
            raise

    def run(self, src: torch.Tensor, dst: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
        # a repartition copies bytes: any dtype of the relation's element size will do
        esize = B.DTYPE_SIZE[self.src.dtype]
        for t, what in ((src, "source"), (dst, "destination")):
            if isinstance(t, torch.Tensor) and t.element_size() != esize:
                raise ValueError("%s: %d-byte elements, the relation has %d-byte elements" %
                                 (what, t.element_size(), esize))
        sptr, dptr = check_buffers([(src, self.src.nbytes, None, "source"),
                                    (dst, self.dst.nbytes, None, "destination")])
        B.ja_repart_run(self.rp, sptr, dptr, stream_handle(stream))

    def close(self):
        if self.rp:
            B.ja_repart_destroy(self.rp)
            self.rp = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceJoin:
    """The join of one spec over a grid of fixed interval counts, run on the
    device from split points in device memory (ja_djoin_*).

    `counts` maps every letter to its number of intervals and `extents` to
    its extent.  ``run(splits)`` enqueues the join; ``splits`` is a device
    int64 tensor holding, letter after letter (letter order), each letter's
    intervals + 1 split points.  The records, segment offsets and
    [n_tuples, n_segs, status] stay in device memory (``rec``, ``seg_off``,
    ``counts``)."""

    def __init__(self, einsum: str, op: str, counts: Dict[str, int], extents: Dict[str, int], params: str = "",
                 device="cuda", stream: Optional[torch.cuda.Stream] = None):
        self.spec = B.ja_spec_create(einsum, op, params)
        self.dj = None
        try:
            self.letters = B.ja_spec_letters(self.spec)
            self.dj = B.ja_djoin_create(self.spec, [extents[c] for c in self.letters],
                                        [counts[c] for c in self.letters])
            tb, wb, self.max_tuples, self.max_segs, self.n_splits = B.ja_djoin_device_bytes(self.dj)
            self.table = _table(tb, device)
            B.ja_djoin_upload(self.dj, self.table.data_ptr(), self.table.numel(), stream_handle(stream))
            self.workspace = torch.empty(max(wb, 256), dtype=torch.uint8, device=device)
            nl = len(self.letters)
            self.rec = torch.empty(max(self.max_tuples * nl, 1), dtype=torch.int32, device=device)
            self.seg_off = torch.empty(self.max_segs + 1, dtype=torch.int64, device=device)
            self.counts = torch.empty(3, dtype=torch.int64, device=device)
        except Exception:
            self.close()
            raise

    def run(self, splits: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
        if splits.dtype != torch.int64 or not splits.is_cuda or splits.numel() != self.n_splits:
            raise ValueError("splits: a device int64 tensor of %d split points" % self.n_splits)
        B.ja_djoin_run(self.dj, splits.data_ptr(), self.rec.data_ptr(), self.seg_off.data_ptr(),
                       self.counts.data_ptr(), self.workspace.data_ptr(), stream_handle(stream))

    def result(self):
        """(records [n, letters] int32, segment offsets [nseg + 1] int64,
        status) copied to the host (synchronises)."""
        nt, ns, status = (int(v) for v in self.counts.cpu())
        nl = len(self.letters)
        rec = self.rec[: nt * nl].cpu().numpy().reshape(nt, nl)
        return rec, self.seg_off[: ns + 1].cpu().numpy(), status

    def close(self):
        if self.dj:
            B.ja_djoin_destroy(self.dj)
            self.dj = None
        if self.spec:
            B.ja_spec_destroy(self.spec)
            self.spec = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceAttention:
    """Attention over packed sequences whose ends are device data
    (ja_dattn_*, spec params with "packed=device"): ``run(splits, Q, K, V,
    O)`` enqueues the device-side join, the kernels that build the attention
    tables and the attention kernel on one stream.  ``splits`` holds every
    letter's split points (letter order), those of s and t being the sequence
    ends.  ``counts`` keeps the join's [n_tuples, n_segs, status]."""

    def __init__(self, einsum: str, counts: Dict[str, int], extents: Dict[str, int],
                 params: str = "packed=device;causal=s,t", dtype: int = JA_BF16, device="cuda",
                 stream: Optional[torch.cuda.Stream] = None):
        self.spec = B.ja_spec_create(einsum, "attention", params)
        self.da = None
        try:
            self.letters = B.ja_spec_letters(self.spec)
            self.da = B.ja_dattn_create(self.spec, [extents[c] for c in self.letters],
                                        [counts[c] for c in self.letters], dtype)
            # Q, K, V, O hold every element of their letters' extents (their
            # blocks tile them whatever the sequence ends)
            esize = B.DTYPE_SIZE[dtype]
            self._tdtype = TORCH_DTYPE[dtype]
            lhs, out = einsum.split("->")
            self._nbytes = [esize * int(np.prod([extents[c] for c in x])) for x in lhs.split(",") + [out]]
            tb, wb, self.n_splits = B.ja_dattn_device_bytes(self.da)
            self.table = torch.empty(max(tb, 256), dtype=torch.uint8, device=device)
            B.ja_dattn_upload(self.da, self.table.data_ptr(), self.table.numel(), stream_handle(stream))
            self.workspace = torch.empty(max(wb, 256), dtype=torch.uint8, device=device)
            self.counts = torch.zeros(3, dtype=torch.int64, device=device)
        except Exception:
            self.close()
            raise

    def run(self, splits: torch.Tensor, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor,
            stream: Optional[torch.cuda.Stream] = None):
        if splits.dtype != torch.int64 or not splits.is_cuda or splits.numel() != self.n_splits:
            raise ValueError("splits: a device int64 tensor of %d split points" % self.n_splits)
        q, k, v, o = check_buffers([(t, n, self._tdtype, w) for t, n, w in zip((Q, K, V, O), self._nbytes, "QKVO")])
        B.ja_dattn_run(self.da, splits.data_ptr(), q, k, v, o, self.counts.data_ptr(), self.workspace.data_ptr(),
                       stream_handle(stream))

    def close(self):
        if self.da:
            B.ja_dattn_destroy(self.da)
            self.da = None
        if self.spec:
            B.ja_spec_destroy(self.spec)
            self.spec = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
