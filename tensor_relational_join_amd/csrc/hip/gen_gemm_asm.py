"""Write gemm_asm.inc: the contraction's K loop as inline assembly.

The direct-to-LDS contraction kernel (gemm.hip) multiplies one 32-wide stage
per step: 32 (or 16) v_mfma_f32_16x16x32 per wavefront, the next stage's
fragment reads from LDS and the refill loads of a freed stage buffer.  The
matrix pipe stays fed only if those reads and loads are threaded between the
MFMAs one or two at a time; the compiler either issues them in blocks or,
with the accumulators and both fragment sets live (about 250 registers),
spills.  So the loop is written out here: accumulators are asm operands in
AGPRs, fragments live in fixed VGPRs v0 .. v(2 S - 1) that the statement
clobbers (S = 4 (FM + FN) per set), and the schedule is exactly the
instruction order below.

One statement per instance (fragment rows FM, columns FN, B layout, dtype)
runs the steps of one run of a tile:
  head  -- optionally, the tile's first three steps, which may also leave the
           previous tile's output stores in flight (see statement());
  run   -- n1 steps that each refill one stage: wait for the stage read
           next (vmcnt: two later stages may stay in flight), barrier, MFMAs
           with the reads and loads between them, then advance the LDS read
           addresses, the refill's LDS bases and global offsets;
  drain -- n2 steps with no refill (the last stages of a tile), each waiting
           for no more than its own stage.
The statement first re-reads the current stage's fragments (the compiler
owns the fixed VGPRs between statements) and ends with enough wait states for
a VALU read of the accumulators.  Run as a script (build.py does) it writes
the file given as its argument.
"""
import sys

NS = 4  # stage buffers in the ring


def _read_ops(fm, fn, b_tr, base):
    """LDS reads of one fragment set at register base: A rows (16-byte reads), then B."""
    ops = []
    for i in range(fm):
        r = base + 4 * i
        ops.append("ds_read_b128 v[%d:%d], %%[ra] offset:%d" % (r, r + 3, i * 1024))
    for j in range(fn):
        r = base + 4 * fm + 4 * j
        if b_tr:  # k strided: two transposing 8-byte reads (k, k + 4) per fragment
            ops.append("ds_read_b64_tr_b16 v[%d:%d], %%[rb%d]" % (r, r + 1, 2 * j))
            ops.append("ds_read_b64_tr_b16 v[%d:%d], %%[rb%d]" % (r + 2, r + 3, 2 * j + 1))
        else:
            ops.append("ds_read_b128 v[%d:%d], %%[rb0] offset:%d" % (r, r + 3, j * 1024))
    return ops


def _mfmas(fm, fn, f16, base):
    name = "v_mfma_f32_16x16x32_%s" % ("f16" if f16 else "bf16")
    out = []
    for i in range(fm):
        for j in range(fn):
            a = base + 4 * i
            b = base + 4 * fm + 4 * j
            acc = "%%[c%d_%d]" % (i, j)
            # operands swapped: each lane ends up with four adjacent output columns
            out.append("%s %s, v[%d:%d], v[%d:%d], %s" % (name, acc, b, b + 3, a, a + 3, acc))
    return out


def _dmas(pa, pb):
    ops = []
    for j in range(pa):
        ops.append(["s_add_u32 m0, %%[ma], %d" % (j * 1024), "buffer_load_dwordx4 %%[va%d], %%[rsa], %%[sa] offen lds" % j])
    for j in range(pb):
        ops.append(["s_add_u32 m0, %%[mb], %d" % (j * 1024), "buffer_load_dwordx4 %%[vb%d], %%[rsb], %%[sb] offen lds" % j])
    return ops


def _advance(nrb, sa_stage, sb_stage, refill):
    """Point the read addresses at the next stage buffer (and the refill bases at the next freed one)."""
    neg_a = -(NS - 1) * sa_stage & 0xFFFFFFFF
    neg_b = -(NS - 1) * sb_stage & 0xFFFFFFFF
    # one literal per scalar instruction: the step, then the wrap-around step if SCC
    def sel(cmp):
        return [cmp, "s_mov_b32 %%[t0], %d" % sa_stage, "s_cmov_b32 %%[t0], 0x%x" % neg_a,
                "s_mov_b32 %%[t1], %d" % sb_stage, "s_cmov_b32 %%[t1], 0x%x" % neg_b]
    out = ["s_add_u32 %[ph], %[ph], 1", "s_cmp_eq_u32 %%[ph], %d" % NS, "s_cselect_b32 %[ph], 0, %[ph]"]
    out += sel("s_cmp_eq_u32 %[ph], 0")
    out += ["v_add_u32 %[ra], %[t0], %[ra]"]
    out += ["v_add_u32 %%[rb%d], %%[t1], %%[rb%d]" % (k, k) for k in range(nrb)]
    if refill:
        # the buffer refilled next is the one before the buffer read next
        out += ["s_add_u32 %[sa], %[sa], %[ia]", "s_add_u32 %[sb], %[sb], %[ib]"] + sel("s_cmp_eq_u32 %[ph], 1")
        out += ["s_add_u32 %[ma], %[ma], %[t0]", "s_add_u32 %[mb], %[mb], %[t1]"]
    return out


def _step(fm, fn, b_tr, f16, cur, nxt, pa, pb, refill, vm=None, extra=0):
    """One step; vm = stages that may stay in flight past the one read next,
    extra = further memory operations issued after that stage (a previous
    tile's output stores) that may stay in flight too."""
    ps = pa + pb
    if vm is None:
        vm = NS - 2 if refill else 0
    out = ["s_waitcnt vmcnt(%d)" % (vm * ps + extra), "s_waitcnt lgkmcnt(0)", "s_barrier"]
    mf = _mfmas(fm, fn, f16, cur)
    reads = _read_ops(fm, fn, b_tr, nxt)
    dmas = _dmas(pa, pb) if refill else []
    m = len(mf)
    slot_r = {}
    for k in range(len(reads)):
        slot_r.setdefault(k * m // len(reads), []).append(reads[k])
    slot_d = {}  # loads early, after the odd MFMAs, so they have the most time to land
    for k in range(len(dmas)):
        slot_d.setdefault(2 * k + 1, []).extend(dmas[k])
    for q in range(m):
        out.append(mf[q])
        out += slot_r.get(q, [])
        out += slot_d.get(q, [])
    return out


def statement(fm, fn, b_tr, f16, bm, bn):
    """n1 steps that refill a stage each, then n2 steps that refill nothing.

    With nh != 0 (the caller guarantees n1 >= NS - 1) the first NS - 1 steps
    are head steps: the tile's first NS stages were loaded before the
    previous tile's full-tile epilogue, which issued nh memory operations
    per fragment pair and lane (a store; or a residual load and a store), so
    the stage a head step reads is followed in issue order by those
    nh * fm * fn / 2 operations as well as the usual NS - 2 stages, and the
    head steps do not wait for the epilogue's stores to complete."""
    s = 4 * (fm + fn)
    stores = fm * fn // 2
    pa = bm * 32 // 8 // 64 // 8
    pb = bn * 32 // 8 // 64 // 8
    nrb = 2 * fn if b_tr else 1
    sa_stage, sb_stage = bm * 64, bn * 64  # bytes of one stage's A and B tile
    body = ["s_nop 4"]  # the compiler may have just written the accumulators
    body += _read_ops(fm, fn, b_tr, 0)
    body += _advance(nrb, sa_stage, sb_stage, False)
    body += ["s_cmp_eq_u32 %[n1], 0", "s_cbranch_scc1 3f", "s_cmp_eq_u32 %[nh], 0", "s_cbranch_scc1 1f",
             "s_cmp_eq_u32 %[nh], 1", "s_cbranch_scc0 7f"]
    # head steps (NS - 1 = 3 of them: fragment sets 0, 1, 0), then the refill
    # loop's second half (current set 1) or the drain from set 1
    assert NS - 1 == 3
    for kind in (1, 2):
        if kind == 2:
            body += ["7:"]
        for k in range(NS - 1):
            cur = 0 if k % 2 == 0 else s
            body += _step(fm, fn, b_tr, f16, cur, s - cur, pa, pb, True, extra=kind * stores)
            body += _advance(nrb, sa_stage, sb_stage, True) + ["s_sub_u32 %[n1], %[n1], 1"]
        body += ["s_cmp_eq_u32 %[n1], 0", "s_cbranch_scc1 4f", "s_branch 8f"]
    # refill steps, current fragments in set 0 then set 1
    body += ["1:"] + _step(fm, fn, b_tr, f16, 0, s, pa, pb, True) + _advance(nrb, sa_stage, sb_stage, True)
    body += ["s_sub_u32 %[n1], %[n1], 1", "s_cmp_eq_u32 %[n1], 0", "s_cbranch_scc1 4f"]
    body += ["8:"] + _step(fm, fn, b_tr, f16, s, 0, pa, pb, True) + _advance(nrb, sa_stage, sb_stage, True)
    body += ["s_sub_u32 %[n1], %[n1], 1", "s_cmp_eq_u32 %[n1], 0", "s_cbranch_scc0 1b"]
    # The last NS steps of a tile (n2 == NS after a run that reaches the end):
    # step k may leave the NS - 2 - k stages loaded after the one it reads in
    # flight.  Any other n2 (a tile of fewer than NS stages) waits for all.
    def drain_exact(first):
        out = []
        for k in range(NS):
            cur = first if k % 2 == 0 else s - first
            out += _step(fm, fn, b_tr, f16, cur, s - cur, pa, pb, False, max(0, NS - 2 - k))
            out += _advance(nrb, sa_stage, sb_stage, False)
        return out
    def drain_loop(first, lab):
        other = s - first
        out = ["%d:" % lab] + _step(fm, fn, b_tr, f16, first, other, pa, pb, False) + _advance(nrb, sa_stage, sb_stage, False)
        out += ["s_sub_u32 %[n2], %[n2], 1", "s_cmp_eq_u32 %[n2], 0", "s_cbranch_scc1 6f"]
        out += _step(fm, fn, b_tr, f16, other, first, pa, pb, False) + _advance(nrb, sa_stage, sb_stage, False)
        out += ["s_sub_u32 %[n2], %[n2], 1", "s_cmp_eq_u32 %[n2], 0", "s_cbranch_scc0 %db" % lab, "s_branch 6f"]
        return out
    # drain starting from set 0
    body += ["3:", "s_cmp_eq_u32 %[n2], 0", "s_cbranch_scc1 6f", "s_cmp_eq_u32 %%[n2], %d" % NS, "s_cbranch_scc0 2f"]
    body += drain_exact(0) + ["s_branch 6f"]
    body += drain_loop(0, 2)
    # drain starting from set 1
    body += ["4:", "s_cmp_eq_u32 %[n2], 0", "s_cbranch_scc1 6f", "s_cmp_eq_u32 %%[n2], %d" % NS, "s_cbranch_scc0 5f"]
    body += drain_exact(s) + ["s_branch 6f"]
    body += drain_loop(s, 5)
    body += ["6:", "s_waitcnt lgkmcnt(0)", "s_nop 7", "s_nop 7", "s_nop 4"]
    outs = ['[c%d_%d] "+a"(acc[%d][%d])' % (i, j, i, j) for i in range(fm) for j in range(fn)]
    outs += ['[n1] "+s"(n1)', '[n2] "+s"(n2)', '[ph] "+s"(ph)', '[ra] "+v"(ra)']
    outs += ['[rb%d] "+v"(rb[%d])' % (k, k) for k in range(nrb)]
    outs += ['[t0] "=&s"(t0)', '[t1] "=&s"(t1)']
    outs += ['[sa] "+s"(sa)', '[sb] "+s"(sb)', '[ma] "+s"(ma)', '[mb] "+s"(mb)']
    ins = ['[rsa] "s"(rsa)', '[rsb] "s"(rsb)', '[ia] "s"(ia)', '[ib] "s"(ib)', '[nh] "s"(nh)']
    ins += ['[va%d] "v"(va[%d])' % (j, j) for j in range(pa)]
    ins += ['[vb%d] "v"(vb[%d])' % (j, j) for j in range(pb)]
    clob = ['"v%d"' % r for r in range(2 * s)] + ['"m0"', '"scc"', '"memory"']
    lines = "\n".join('        "%s\\n"' % l for l in body)
    return "    asm volatile(\n%s\n        : %s\n        : %s\n        : %s);\n" % (
        lines, ",\n          ".join(outs), ",\n          ".join(ins), ", ".join(clob))


def emit():
    out = ["// Generated by gen_gemm_asm.py; do not edit.", "",
           "template <int FM, bool KN, bool F16>", "struct GemmAsm;", ""]
    for fm, bm in ((8, 256), (4, 128)):
        fn, bn = 4, 256
        for b_tr in (True, False):
            for f16 in (False, True):
                nrb = 2 * fn if b_tr else 1
                pa = bm * 32 // 8 // 64 // 8
                pb = bn * 32 // 8 // 64 // 8
                out.append("template <>")
                out.append("struct GemmAsm<%d, %s, %s> {" % (fm, "true" if b_tr else "false", "true" if f16 else "false"))
                out.append("    static constexpr int PA = %d, PB = %d, NRB = %d, STORES = %d;" % (pa, pb, nrb, fm * fn // 2))
                out.append("    __device__ __forceinline__ static void steps(f32x4_t (&acc)[%d][%d], uint32_t n1, uint32_t n2, "
                           "uint32_t ph, uint32_t ra, uint32_t (&rb)[%d], i32x4_t rsa, i32x4_t rsb, const uint32_t (&va)[%d], "
                           "const uint32_t (&vb)[%d], uint32_t sa, uint32_t sb, uint32_t ia, uint32_t ib, uint32_t ma, "
                           "uint32_t mb, uint32_t nh) {" % (fm, fn, nrb, pa, pb))
                out.append("    uint32_t t0, t1;")
                out.append(statement(fm, fn, b_tr, f16, bm, bn) + "    }")
                out.append("};")
                out.append("")
    return "\n".join(out)


if __name__ == "__main__":
    with open(sys.argv[1], "w") as f:
        f.write(emit())
