"""ja_einsum_noalloc (the one-shot join-agg that allocates no device memory:
plan tables and run scratch in the library's static device array) against
ja_einsum (the same with a caller workspace), through the C ABI: two calls in
a row on each operator, the second with a smaller input, outputs compared
bit for bit (the same kernels run on the same inputs)."""
import numpy as np
import pytest

from tensor_relational_join_amd import synth

pytestmark = pytest.mark.gpu


def _eq(n, q):
    base, extra = divmod(n, q)
    p = [0]
    for i in range(q):
        p.append(p[-1] + base + (i < extra))
    return p


def _both(einsum, op, sp, params, arrays):
    """Run ja_einsum and ja_einsum_noalloc on the same device inputs; return
    both outputs as int16 bit patterns on the host."""
    import torch

    from tensor_relational_join_amd import binding as B
    from tensor_relational_join_amd.device import relation_for

    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    s = B.ja_spec_create(einsum, op, params)
    try:
        letters = B.ja_spec_letters(s)
        d = B.ja_decomp_create(s, [sp[c][-1] for c in letters], [len(sp[c]) - 1 for c in letters],
                               [sp[c] for c in letters])
        try:
            rels = [relation_for(x, sp, B.JA_BF16) for x in ins]
            orel = relation_for(out, sp, B.JA_BF16)
            import oracle as orc

            dev = [torch.from_numpy(orc.Relation(r.shape, r.splits).pack(a).view(np.int16).ravel()).cuda()
                   for r, a in zip(rels, arrays)]
            ptrs = [t.data_ptr() for t in dev]
            stream = torch.cuda.current_stream().cuda_stream
            n_out = orel.nbytes // 2
            want = torch.full((n_out,), -1, dtype=torch.int16, device="cuda")
            got = torch.full((n_out,), -2, dtype=torch.int16, device="cuda")
            wsb = B.ja_einsum_workspace_bytes(s, d, rels, orel)
            assert wsb <= B.JA_NOALLOC_SCRATCH_BYTES
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
            B.ja_einsum(s, d, rels, ptrs, orel, want.data_ptr(), ws.data_ptr(), ws.numel(), stream)
            B.ja_einsum_noalloc(s, d, rels, ptrs, orel, got.data_ptr(), stream)
            torch.cuda.synchronize()
            return want.cpu().numpy(), got.cpu().numpy()
        finally:
            B.ja_decomp_destroy(d)
    finally:
        B.ja_spec_destroy(s)


def test_noalloc_contraction_two_calls():
    for seed, (M, K, N), q in ((1, (1024, 512, 2752), 2), (2, (256, 128, 512), 1)):
        sp = {"b": _eq(M, q), "d": _eq(K, 2), "f": _eq(N, q)}
        X = synth.normal_bf16(40 + seed, 0, (M, K))
        W = synth.normal_bf16(40 + seed, 1, (K, N), std=0.05)
        want, got = _both("bd,df->bf", "contract", sp, "", [X, W])
        assert np.array_equal(want, got)
        assert np.all(want != -1)


def test_noalloc_attention_two_calls():
    """bf16 attention uses run scratch as well (its range-check flags): the
    second, smaller call finds the first call's flags in the array."""
    for seed, (H, S) in ((3, (4, 512)), (4, (2, 200))):
        sp = {"b": [0, 1], "h": _eq(H, H), "s": _eq(S, -(-S // 128)), "t": _eq(S, -(-S // 128)), "d": [0, 128]}
        Q = synth.normal_bf16(50 + seed, 0, (1, H, S, 128))
        K = synth.normal_bf16(50 + seed, 1, (1, H, S, 128))
        V = synth.normal_bf16(50 + seed, 2, (1, H, S, 128))
        want, got = _both("bhsd,bhtd,bhtd->bhsd", "attention", sp, "causal=s,t", [Q, K, V])
        assert np.array_equal(want, got)
        assert np.all(want != -1)
