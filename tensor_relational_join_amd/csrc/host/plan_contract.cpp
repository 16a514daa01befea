// plan_contract.cpp -- the contraction planner: the fused GEMM-shaped tables
// (output tiles of every segment, segments, tuples) of a contraction's
// join-agg spec ("Every Kernel Is a Join", paperpeel full text, section 3.2,
// Examples 3.8 and 3.9: block products whose partial results are SUM-aggregated
// per output block).
#include <algorithm>
#include <climits>
#include <cmath>

#include "plan_internal.h"

namespace ja {
namespace {

// Split an operand's letters into role runs.  Returns false unless the
// operand is [batch run][first run][second run] with the two named roles in
// either order; `first_is` reports which role came first.
bool runs(const std::string& op, const std::string& batch, const std::string& r1, const std::string& r2,
          bool& r1_first) {
    size_t nb = batch.size();
    if (op.substr(0, nb) != batch) return false;
    std::string rest = op.substr(nb);
    if (rest == r1 + r2) {
        r1_first = true;
        return true;
    }
    if (rest == r2 + r1) {
        r1_first = false;
        return true;
    }
    return false;
}

}  // namespace

ja_status plan_contract(ja_plan* p, const ja_spec* s, const ja_decomp* d, const ja_tuples& t,
                        const ja_relation_desc* const* in, const ja_relation_desc* out) {
    Rel A, B, C;
    ja_status st;
    if ((st = rel_from_desc(in[0], A)) || (st = rel_from_desc(in[1], B)) || (st = rel_from_desc(out, C))) return st;
    const bool swig = s->epilogue == JA_EPI_SWIGLU;
    // With the SwiGLU epilogue the kernel computes the contraction into the
    // output's letters followed by the pair letter (whole, extent 2): element
    // e of that layout is member e % 2 of the pair written to element e / 2
    // of the real output, so its block offsets are twice the output's.
    const std::string &sa = s->ins[0], &sb = s->ins[1];
    const std::string sc = swig ? s->out + s->pair : s->out;
    if ((st = match_rel(C, s->out, s, d, "output"))) return st;
    if (swig) {
        const int l = s->letter_index(s->pair);
        if (d->ext[l] != 2 || d->sp[l].size() != 2)
            return fail(JA_ERR_DECOMP, "the (gate, up) pair letter must have extent 2 and one interval");
    }
    if (s->epilogue != JA_EPI_NONE) {
        if (A.dtype == JA_F32 || C.dtype != A.dtype)
            return fail(JA_ERR_DTYPE, "a contraction with an epilogue takes and writes bf16 or f16");
        if (s->epilogue == JA_EPI_ADD) {
            Rel R;
            if ((st = rel_from_desc(in[2], R)) || (st = match_rel(R, s->out, s, d, "residual"))) return st;
            if (R.dtype != C.dtype) return fail(JA_ERR_DTYPE, "the residual must have the output's dtype");
        }
    }
    p->epilogue = s->epilogue;
    if (A.dtype != B.dtype) return fail(JA_ERR_DTYPE, "contract operands must share a dtype");
    if (A.dtype == JA_F32) {
        if (C.dtype != JA_F32) return fail(JA_ERR_DTYPE, "f32 contraction writes f32");
    } else if (A.dtype == JA_BF16 || A.dtype == JA_F16) {
        if (C.dtype != A.dtype && C.dtype != JA_F32)
            return fail(JA_ERR_DTYPE, "a 16-bit contraction writes its input format or f32");
    } else {
        return fail(JA_ERR_DTYPE, "contract supports f32, bf16 and f16 operands");
    }
    const bool h16 = A.dtype != JA_F32;  // bf16 or f16: the MFMA kernels
    // roles of the letters: batch (A, B, C), M (A, C), N (B, C), K (A, B)
    std::string batch, M, N, K;
    for (char c : sc) {
        bool ia = sa.find(c) != std::string::npos, ib = sb.find(c) != std::string::npos;
        if (ia && ib) batch.push_back(c);
    }
    for (char c : sc)
        if (batch.find(c) == std::string::npos) (sa.find(c) != std::string::npos ? M : N).push_back(c);
    for (char c : sa)
        if (sc.find(c) == std::string::npos) K.push_back(c);
    // M and N in the output's order; K in A's order
    std::string Mo, No;
    for (char c : sc) {
        if (M.find(c) != std::string::npos) Mo.push_back(c);
        if (N.find(c) != std::string::npos) No.push_back(c);
    }
    bool a_m_first = true, b_k_first = true;
    if (sc != batch + Mo + No || !runs(sa, batch, Mo, K, a_m_first) || !runs(sb, batch, K, No, b_k_first))
        return fail(JA_ERR_UNSUPPORTED,
                    "contract needs operands laid out as [batch][rows][cols] runs with matching letter orders");
    // An operand of two letters (no batch letter) may be blocked coarser than
    // the decomposition: a tuple then reads its sub-box of the block in place
    // (offset inside the block, the block's row length as leading dimension),
    // so a refinement of an operand's blocking needs no repartition.
    const bool a_sub = batch.empty() && sa.size() == 2, b_sub = batch.empty() && sb.size() == 2;
    if ((st = a_sub ? match_rel_coarse(A, sa, s, d, "operand A") : match_rel(A, sa, s, d, "operand A")) ||
        (st = b_sub ? match_rel_coarse(B, sb, s, d, "operand B") : match_rel(B, sb, s, d, "operand B")))
        return st;
    // a tuple's sub-box of a two-letter operand: element offset, leading
    // dimension (the block's inner extent) and the sub-box's span (outer
    // interval extent times the leading dimension)
    auto sub_box = [&](const Rel& X, const std::string& xs, const int32_t* rec, int64_t& off, int64_t& ld,
                       int64_t& span) {
        const int l0 = s->letter_index(xs[0]), l1 = s->letter_index(xs[1]);
        const int64_t lo0 = d->sp[l0][rec[l0]], lo1 = d->sp[l1][rec[l1]];
        int64_t key[2] = {X.find(0, lo0), X.find(1, lo1)};
        ld = X.ext(1, key[1]);
        off = X.blk_off[X.block_index(key)] + (lo0 - X.sp[0][key[0]]) * ld + (lo1 - X.sp[1][key[1]]);
        span = (d->sp[l0][rec[l0] + 1] - lo0) * ld;
    };
    p->a_layout = a_m_first ? JA_A_MK : JA_A_KM;
    p->b_layout = b_k_first ? JA_B_KN : JA_B_NK;
    p->in_dtype = A.dtype;
    p->out_dtype = C.dtype;
    const int TM = h16 ? GEMM_BF16_TM : GEMM_F32_TM;
    const int TN = h16 ? GEMM_BF16_TN : GEMM_F32_TN;

    const int64_t nt = t.count(), nseg = (int64_t)t.seg.size() - 1;
    std::vector<GemmTuple> tuples(nt);
    std::vector<GemmSeg> segs(nseg), usegs(nt);
    std::vector<GemmTile> tiles, utiles;
    std::vector<AggTile> atiles;
    std::vector<AggSeg> asegs(nseg);
    std::vector<int64_t> poff(nt);
    int64_t part = 0;
    const int64_t lim = ((int64_t)1 << 31) - 1;
    for (int64_t i = 0; i < nt; ++i) {
        const int32_t* rec = &t.rec[i * t.nl];
        int64_t nb = extent_of(d, s, rec, batch), m = extent_of(d, s, rec, Mo), n = extent_of(d, s, rec, No),
                k = extent_of(d, s, rec, K);
        if (m > lim || n > lim || k > lim) return fail(JA_ERR_UNSUPPORTED, "block extent beyond 2^31");
        GemmTuple& g = tuples[i];
        g.a_off = A.blk_off[block_of(A, sa, s, rec)];
        g.b_off = B.blk_off[block_of(B, sb, s, rec)];
        g.a_bstride = m * k;
        g.b_bstride = k * n;
        g.K = (int32_t)k;
        g.lda = (int32_t)(a_m_first ? k : m);
        g.ldb = (int32_t)(b_k_first ? n : k);
        if (a_sub) {  // (with the decomposition's own blocking this gives the values above)
            int64_t ld, span;
            sub_box(A, sa, rec, g.a_off, ld, span);
            if (ld > lim) return fail(JA_ERR_UNSUPPORTED, "block extent beyond 2^31");
            g.lda = (int32_t)ld;
            g.a_bstride = span;
        }
        if (b_sub) {
            int64_t ld, span;
            sub_box(B, sb, rec, g.b_off, ld, span);
            if (ld > lim) return fail(JA_ERR_UNSUPPORTED, "block extent beyond 2^31");
            g.ldb = (int32_t)ld;
            g.b_bstride = span;
        }
        g.pad = 0;
        // unfused: every tuple is its own segment writing an f32 partial block
        GemmSeg& u = usegs[i];
        u.c_off = part;
        u.c_bstride = m * n;
        u.M = (int32_t)m;
        u.N = (int32_t)n;
        u.ldc = (int32_t)n;
        u.t_begin = (int32_t)i;
        u.t_end = (int32_t)i + 1;
        u.nst = (int32_t)((k + GEMM_DMA_BK - 1) / GEMM_DMA_BK);
        poff[i] = part;
        part += nb * m * n;
        for (int32_t b = 0; b < nb; ++b)
            for (int32_t m0 = 0; m0 < m; m0 += TM)
                for (int32_t n0 = 0; n0 < n; n0 += TN) utiles.push_back({(int32_t)i, m0, n0, b});
    }
    for (int64_t sg = 0; sg < nseg; ++sg) {
        const int32_t* rec = &t.rec[t.seg[sg] * t.nl];
        int64_t nb = extent_of(d, s, rec, batch), m = extent_of(d, s, rec, Mo), n = extent_of(d, s, rec, No);
        GemmSeg& g = segs[sg];
        g.c_off = C.blk_off[block_of(C, s->out, s, rec)] * (swig ? 2 : 1);
        g.c_bstride = m * n;
        g.M = (int32_t)m;
        g.N = (int32_t)n;
        g.ldc = (int32_t)n;
        g.t_begin = (int32_t)t.seg[sg];
        g.t_end = (int32_t)t.seg[sg + 1];
        int64_t nst = 0;
        for (int32_t i = g.t_begin; i < g.t_end; ++i) nst += (tuples[i].K + GEMM_DMA_BK - 1) / GEMM_DMA_BK;
        if (nst > lim) return fail(JA_ERR_UNSUPPORTED, "contracted extent beyond 2^31 stages");
        g.nst = (int32_t)nst;
        // grouped order: GEMM_GROUP_M row tiles, then every column tile, so a
        // contiguous run of the list forms a compact block of output tiles
        const int32_t mt = (int32_t)((m + TM - 1) / TM), ntl = (int32_t)((n + TN - 1) / TN);
        for (int32_t b = 0; b < nb; ++b)
            for (int32_t mg = 0; mg < mt; mg += GEMM_GROUP_M)
                for (int32_t nj = 0; nj < ntl; ++nj)
                    for (int32_t mi = mg; mi < std::min(mt, mg + GEMM_GROUP_M); ++mi)
                        tiles.push_back({(int32_t)sg, mi * TM, nj * TN, b});
        AggSeg& a = asegs[sg];
        a.out_off = g.c_off;
        if (nb * m * n > lim) return fail(JA_ERR_UNSUPPORTED, "output block beyond 2^31 elements");
        a.nelem = (int32_t)(nb * m * n);
        a.t_begin = g.t_begin;
        a.t_end = g.t_end;
        a.pad = 0;
        for (int32_t e0 = 0; e0 < a.nelem; e0 += AGG_CHUNK) atiles.push_back({(int32_t)sg, e0});
    }
    if ((int64_t)tiles.size() > lim || (int64_t)utiles.size() > lim) return fail(JA_ERR_UNSUPPORTED, "too many tiles");
    if (h16) {
        // the MFMA kernel moves 8 bf16 (16 bytes) at a time along every contiguous axis
        for (const GemmTuple& g : tuples) {
            bool ok = g.K % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.a_off % 8 == 0 && g.b_off % 8 == 0 &&
                      g.a_bstride % 8 == 0 && g.b_bstride % 8 == 0;
            if (!ok) return fail(JA_ERR_UNSUPPORTED, "a 16-bit contraction needs block extents that are multiples of 8");
        }
        for (const GemmSeg& g : segs)
            if ((!a_m_first && g.M % 8) || (b_k_first && g.N % 8))
                return fail(JA_ERR_UNSUPPORTED, "a 16-bit contraction needs block extents that are multiples of 8");
        // the MFMA kernel addresses each operand matrix with 32-bit buffer byte offsets
        for (const GemmTuple& g : tuples)
            if (g.a_bstride >= ((int64_t)1 << 30) || g.b_bstride >= ((int64_t)1 << 30))
                return fail(JA_ERR_UNSUPPORTED, "a 16-bit contraction operand matrix must hold fewer than 2^30 elements");
    }
    p->partial_elems = part;
    p->tiles_off = put(p->table, tiles);
    p->ntiles = (int32_t)tiles.size();
    p->segs_off = put(p->table, segs);
    p->tuples_off = put(p->table, tuples);
    p->utiles_off = put(p->table, utiles);
    p->nutiles = (int32_t)utiles.size();
    p->usegs_off = put(p->table, usegs);
    p->atiles_off = put(p->table, atiles);
    p->natiles = (int32_t)atiles.size();
    p->asegs_off = put(p->table, asegs);
    p->apoff_off = put(p->table, poff);
    return JA_OK;
}

}  // namespace ja
