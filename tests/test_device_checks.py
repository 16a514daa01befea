"""The torch-facing layer refuses buffers a kernel would read or write out of
bounds (wrong dtype, too short, not contiguous, not on the GPU) before any
library call: checked on the CPU with host tensors, so no GPU is touched."""
import pytest
import torch

from tensor_relational_join_amd import binding as B
from tensor_relational_join_amd import device as D


def _op(einsum, splits, dt=B.JA_BF16, out_dt=B.JA_BF16):
    """An Op whose relations are described but whose plan is never built:
    every refusal below must fire before the library is called."""
    op = object.__new__(D.Op)
    lhs, out = einsum.split("->")
    op.in_rels = [D.relation_for(x, splits, dt) for x in lhs.split(",")]
    op.out_rel = D.relation_for(out, splits, out_dt)
    op.plan = op.decomp = op.spec = None
    op.workspace = None
    op.partial_bytes = lambda: 4 * 64 * 64 * 2
    return op


SP = {"i": [0, 32, 64], "j": [0, 64], "k": [0, 64]}


def _bf16(n):
    return torch.zeros(n, dtype=torch.bfloat16)


def test_check_buffer_order_of_refusals():
    with pytest.raises(ValueError, match="dtype"):
        D.check_buffer(torch.zeros(8, dtype=torch.float32), 16, torch.bfloat16, "x")
    with pytest.raises(ValueError, match="needs 64"):
        D.check_buffer(_bf16(8), 64, torch.bfloat16, "x")
    with pytest.raises(ValueError, match="contiguous"):
        D.check_buffer(_bf16(64).view(8, 8).t(), 16, torch.bfloat16, "x")
    with pytest.raises(ValueError, match="GPU"):
        D.check_buffer(_bf16(64), 128, torch.bfloat16, "x")
    with pytest.raises(ValueError, match="torch tensor"):
        D.check_buffer(12345, 16, None, "x")


def test_op_run_refuses_bad_buffers():
    op = _op("ij,jk->ik", SP)
    good = [_bf16(64 * 64), _bf16(64 * 64)]
    with pytest.raises(ValueError, match="input 1: .* bytes, the relation needs 8192"):
        op.run([good[0], _bf16(64 * 63)], _bf16(64 * 64))
    with pytest.raises(ValueError, match="input 0: dtype"):
        op.run([torch.zeros(64 * 64, dtype=torch.float16), good[1]], _bf16(64 * 64))
    with pytest.raises(ValueError, match="2 relations"):
        op.run([good[0]], _bf16(64 * 64))
    with pytest.raises(ValueError, match="output: .* bytes"):
        op.run(good, _bf16(10))
    with pytest.raises(ValueError, match="GPU"):  # everything right except the device
        op.run(good, _bf16(64 * 64))


def test_op_unfused_refuses_bad_partials():
    op = _op("ij,jk->ik", SP)
    good = [_bf16(64 * 64), _bf16(64 * 64)]
    with pytest.raises(ValueError, match="partials: dtype"):
        op.kernel(good, _bf16(2 * 64 * 64))
    with pytest.raises(ValueError, match="partials: .* bytes"):
        op.kernel(good, torch.zeros(100, dtype=torch.float32))
    with pytest.raises(ValueError, match="partials: .* bytes"):
        op.agg(torch.zeros(100, dtype=torch.float32), _bf16(64 * 64))
    with pytest.raises(ValueError, match="output: dtype"):
        op.agg(torch.zeros(2 * 64 * 64, dtype=torch.float32), torch.zeros(64 * 64, dtype=torch.float32))


def test_repart_run_refuses_bad_buffers():
    rp = object.__new__(D.Repart)
    rp.src = B.Relation((64, 64), nblk=(2, 1), dtype=B.JA_BF16)
    rp.dst = B.Relation((64, 64), nblk=(1, 2), dtype=B.JA_BF16)
    rp.rp = None
    with pytest.raises(ValueError, match="source: .* bytes"):
        rp.run(_bf16(100), _bf16(64 * 64))
    with pytest.raises(ValueError, match="destination: 4-byte elements"):
        rp.run(_bf16(64 * 64), torch.zeros(64 * 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):  # raw 16-bit views of the bytes are fine, but not on the host
        rp.run(torch.zeros(64 * 64, dtype=torch.int16), _bf16(64 * 64))


def test_device_attention_refuses_bad_buffers():
    da = object.__new__(D.DeviceAttention)
    da.da = da.spec = None
    da.n_splits = 3
    da._tdtype = torch.bfloat16
    da._nbytes = [2 * 256 * 128] * 4
    splits = torch.zeros(3, dtype=torch.int64)
    with pytest.raises(ValueError, match="splits"):  # splits on the host are refused first
        da.run(splits, *[_bf16(256 * 128)] * 4)
