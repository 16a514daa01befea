// plan.cpp -- join-agg plans: validate relations against a spec and a
// decomposition, run the join, lay out the device tables that drive the fused
// per-tuple kernels, and dispatch them.
//
// The execution follows the three phases of Definition 3.7 ("Every Kernel Is
// a Join", paperpeel full text, section 3.2): every tuple of the join is one
// unit of kernel work; the aggregation of tuples that share an output type is
// fused into the kernel (one workgroup owns each output tile of a segment and
// folds the segment's tuples in ascending order, so no atomics are needed);
// the recompose is in place, since every aggregated block is written straight
// into its slot of the output relation.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>

#include "plan_internal.h"

using namespace ja;

namespace {

// the softmax aggregation writes O rows in [batch-head][query] order
const char* const INNER_UNFUSED =
    "the unfused attention path takes Q, K, V and O with every batch-head letter before the position letter";

ja_status plan_attention(ja_plan* p, const ja_spec* s, const ja_decomp* d, const ja_tuples& t,
                         const ja_relation_desc* const* in, const ja_relation_desc* out) {
    Rel Q, K, V, O;
    ja_status st;
    if ((st = rel_from_desc(in[0], Q)) || (st = rel_from_desc(in[1], K)) || (st = rel_from_desc(in[2], V)) ||
        (st = rel_from_desc(out, O)))
        return st;
    if ((st = match_rel(Q, s->ins[0], s, d, "Q")) || (st = match_rel(K, s->ins[1], s, d, "K")) ||
        (st = match_rel(V, s->ins[2], s, d, "V")) || (st = match_rel(O, s->out, s, d, "O")))
        return st;
    if ((Q.dtype != JA_BF16 && Q.dtype != JA_F16) || K.dtype != Q.dtype || V.dtype != Q.dtype || O.dtype != Q.dtype)
        return fail(JA_ERR_DTYPE, "attention takes and writes bf16 or f16 (one format for Q, K, V and O)");
    p->in_dtype = Q.dtype;
    const std::string& q = s->ins[0];
    const std::string& k = s->ins[1];
    const char cs = s->att_s, ct = s->att_t, cd = q.back();
    // batch-head letters in storage order (all of them, and those stored
    // inside a row: after the position letter)
    std::string batch, kbatch, qin, kin;
    for (size_t i = 0; i + 1 < q.size(); ++i)
        if (q[i] != cs) (i > q.find(cs) ? qin : batch) += q[i];
    batch += qin;
    for (size_t i = 0; i + 1 < k.size(); ++i)
        if (k[i] != ct) (i > k.find(ct) ? kin : kbatch) += k[i];
    kbatch += kin;
    const int64_t D = d->ext[s->letter_index(cd)];
    if (D != ATTN_D) return fail(JA_ERR_UNSUPPORTED, "attention kernel is built for head dimension 128");
    p->scale = (float)(s->has_scale ? s->scale : 1.0 / std::sqrt((double)D));
    p->causal = s->causal ? 1 : 0;
    const int ls = s->letter_index(cs), lt = s->letter_index(ct);
    const int64_t nt = t.count(), nseg = (int64_t)t.seg.size() - 1;
    // packed sequence ends: given, or the cuts of the sequence letter
    const std::vector<int64_t> ends = s->packed_device ? std::vector<int64_t>(d->sp[ls].begin() + 1, d->sp[ls].end())
                                                       : s->packed;
    std::vector<AttnTuple> tuples(nt);
    std::vector<AttnSeg> segs(nseg);
    const int64_t lim = ((int64_t)1 << 31) - 1;
    for (int64_t i = 0; i < nt; ++i) {
        const int32_t* rec = &t.rec[i * t.nl];
        int64_t T = d->sp[lt][rec[lt] + 1] - d->sp[lt][rec[lt]];
        if (T > lim) return fail(JA_ERR_UNSUPPORTED, "key block beyond 2^31");
        AttnTuple& a = tuples[i];
        a.k_off = K.blk_off[block_of(K, s->ins[1], s, rec)];
        a.v_off = V.blk_off[block_of(V, s->ins[2], s, rec)];
        a.kv_bstride = T * extent_of(d, s, rec, kin) * D;
        if (a.kv_bstride > lim) return fail(JA_ERR_UNSUPPORTED, "key block rows beyond 2^31 elements");
        a.T = (int32_t)T;
        a.t_lo = (int32_t)d->sp[lt][rec[lt]];
    }
    struct W {
        AttnTile tile;
        int64_t work;
    };
    std::vector<W> work;
    for (int64_t sg = 0; sg < nseg; ++sg) {
        const int32_t* rec = &t.rec[t.seg[sg] * t.nl];
        int64_t S = d->sp[ls][rec[ls] + 1] - d->sp[ls][rec[ls]];
        int64_t nbh = extent_of(d, s, rec, batch), nkv = extent_of(d, s, rec, kbatch);
        if (S > lim || nbh > lim) return fail(JA_ERR_UNSUPPORTED, "query block beyond 2^31");
        AttnSeg& g = segs[sg];
        // the group letters trail the batch letters, so query batch-head bh
        // of the block reads key-value batch-head bh / rep
        g.rep = (int32_t)(nbh / nkv);
        g.q_hin = (int32_t)extent_of(d, s, rec, qin);
        g.kv_hin = (int32_t)extent_of(d, s, rec, kin);
        g.pad = 0;
        if (g.q_hin > 1 || g.kv_hin > 1) p->att_inner = 1;
        if (S * g.q_hin * D > lim) return fail(JA_ERR_UNSUPPORTED, "query block rows beyond 2^31 elements");
        g.q_off = Q.blk_off[block_of(Q, q, s, rec)];
        g.o_off = O.blk_off[block_of(O, s->out, s, rec)];
        g.q_bstride = S * g.q_hin * D;
        g.S = (int32_t)S;
        g.s_lo = (int32_t)d->sp[ls][rec[ls]];
        g.t_begin = (int32_t)t.seg[sg];
        g.t_end = (int32_t)t.seg[sg + 1];
        for (int32_t bh = 0; bh < nbh; ++bh)
            for (int32_t s0 = 0; s0 < S; s0 += ATTN_TQ) {
                // work estimate: keys visible to the tile's last query row (inside
                // the sequences of the tile's rows when sequences are packed)
                int64_t last = g.s_lo + std::min<int64_t>(S, s0 + ATTN_TQ) - 1, w = 0;
                int64_t klo = 0, khi = INT64_MAX;
                if (!ends.empty()) {
                    auto e1 = std::upper_bound(ends.begin(), ends.end(), (int64_t)g.s_lo + s0);
                    klo = e1 == ends.begin() ? 0 : *(e1 - 1);
                    auto e2 = std::upper_bound(ends.begin(), ends.end(), last);
                    khi = e2 == ends.end() ? ends.back() : *e2;
                }
                for (int32_t k = g.t_begin; k < g.t_end; ++k) {
                    int64_t a = std::max<int64_t>(tuples[k].t_lo, klo);
                    int64_t b = std::min<int64_t>((int64_t)tuples[k].t_lo + tuples[k].T, khi);
                    if (p->causal) b = std::min<int64_t>(b, last + 1);
                    w += std::max<int64_t>(b - a, 0);
                }
                work.push_back({{(int32_t)sg, bh, s0, 0}, w});
            }
    }
    // longest tiles first, so the tail of the launch is short ones
    std::stable_sort(work.begin(), work.end(), [](const W& a, const W& b) { return a.work > b.work; });
    std::vector<AttnTile> tiles;
    tiles.reserve(work.size());
    for (auto& w : work) tiles.push_back(w.tile);
    if ((int64_t)tiles.size() > lim) return fail(JA_ERR_UNSUPPORTED, "too many tiles");
    // Unfused path (ja_kernel / ja_agg): every tuple is a segment of its own
    // writing f32 triples [m, l, -, -, acc[D]] per query row of its block
    // (ATTN_PROW floats, rows in the O block's [bh][s] order) into the
    // partials; the softmax aggregation then folds each segment's tuples.
    std::vector<AttnSeg> usegs(nt);
    std::vector<AttnTile> utiles;
    std::vector<int64_t> poff(nt);
    std::vector<AggSeg> asegs(nseg);
    std::vector<AggTile> atiles;
    int64_t part = 0;
    for (int64_t sg = 0; sg < nseg; ++sg) {
        const AttnSeg& g = segs[sg];
        const int64_t rows = (int64_t)g.S * extent_of(d, s, &t.rec[t.seg[sg] * t.nl], batch);
        if (rows > lim) return fail(JA_ERR_UNSUPPORTED, "query block beyond 2^31 rows");
        for (int32_t k = g.t_begin; k < g.t_end; ++k) {
            AttnSeg u = g;
            u.o_off = part;
            u.t_begin = k;
            u.t_end = k + 1;
            usegs[k] = u;
            poff[k] = part;
            part += rows * ATTN_PROW;
            for (int32_t bh = 0; bh < rows / g.S; ++bh)
                for (int32_t s0 = 0; s0 < g.S; s0 += ATTN_TQ) utiles.push_back({k, bh, s0, 0});
        }
        AggSeg& a = asegs[sg];
        a.out_off = g.o_off;
        a.nelem = (int32_t)rows;
        a.t_begin = g.t_begin;
        a.t_end = g.t_end;
        a.pad = 0;
        for (int32_t r0 = 0; r0 < a.nelem; r0 += SMAX_ROWS) atiles.push_back({(int32_t)sg, r0});
    }
    if ((int64_t)utiles.size() > lim || (int64_t)atiles.size() > lim) return fail(JA_ERR_UNSUPPORTED, "too many tiles");
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
    if (!ends.empty()) {
        std::vector<int32_t> e32(ends.begin(), ends.end());
        p->seq_off = put(p->table, e32);
        p->nseq = (int32_t)e32.size();
    }
    return JA_OK;
}

ja_status plan_rmsnorm(ja_plan* p, const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in,
                       const ja_relation_desc* out) {
    Rel X, G, Y;
    ja_status st;
    if ((st = rel_from_desc(in[0], X)) || (st = rel_from_desc(in[1], G)) || (st = rel_from_desc(out, Y))) return st;
    if ((st = match_rel(X, s->ins[0], s, d, "x")) || (st = match_rel(G, s->ins[1], s, d, "gain")) ||
        (st = match_rel(Y, s->out, s, d, "y")))
        return st;
    if ((X.dtype != JA_BF16 && X.dtype != JA_F16) || G.dtype != X.dtype || Y.dtype != X.dtype)
        return fail(JA_ERR_DTYPE, "rmsnorm takes and writes bf16 or f16 (one format for x, gain and y)");
    p->in_dtype = X.dtype;
    const int64_t D = X.shape[1];
    if (D > 16384) return fail(JA_ERR_UNSUPPORTED, "rmsnorm rows longer than 16384");
    p->nrb = X.nblk(0);
    p->ndb = X.nblk(1);
    p->D = (int32_t)D;
    p->rows = X.shape[0];
    p->eps = (float)s->eps;
    std::vector<int64_t> rsp(X.sp[0]);
    std::vector<NormBlock> blk;
    bool vec = true;  // every row piece 16-byte aligned
    for (int rb = 0; rb < p->nrb; ++rb)
        for (int db = 0; db < p->ndb; ++db) {
            int64_t key[2] = {rb, db};
            NormBlock b{X.blk_off[X.block_index(key)], (int32_t)X.ext(1, db), (int32_t)X.sp[1][db]};
            vec = vec && b.off % 8 == 0 && b.width % 8 == 0;
            blk.push_back(b);
        }
    p->norm_vec = vec ? 1 : 0;
    // rows in registers: equal block widths that are multiples of 512, and a
    // row length the register kernel is instantiated for
    const int64_t W = X.ext(1, 0);
    bool rows_ok = vec && W % 512 == 0 && D % 512 == 0;
    for (int db = 0; db < p->ndb; ++db) rows_ok = rows_ok && X.ext(1, db) == W;
    const int64_t nv = D / 512;
    rows_ok = rows_ok && (nv <= 8 || nv == 10 || nv == 12 || nv == 14 || nv == 16);
    if (rows_ok) {
        p->norm_vec = 2;
        p->norm_w = (int32_t)W;
    }
    p->rsplit_off = put(p->table, rsp);
    p->nblk_off = put(p->table, blk);
    return JA_OK;
}

ja_status plan_zip(ja_plan* p, const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in,
                   const ja_relation_desc* out) {
    Rel A, B, C;
    ja_status st;
    if ((st = rel_from_desc(in[0], A)) || (st = rel_from_desc(in[1], B)) || (st = rel_from_desc(out, C))) return st;
    if ((st = match_rel(A, s->ins[0], s, d, "operand 1")) || (st = match_rel(B, s->ins[1], s, d, "operand 2")) ||
        (st = match_rel(C, s->out, s, d, "output")))
        return st;
    if ((A.dtype != JA_BF16 && A.dtype != JA_F16) || B.dtype != A.dtype || C.dtype != A.dtype)
        return fail(JA_ERR_DTYPE, "elementwise joins take and write bf16 or f16 (one format throughout)");
    p->in_dtype = A.dtype;
    // The three relations are blocked identically, so the 1:1 key join pairs
    // block i of each buffer with block i of the others at identical offsets:
    // the whole join is a zip of the three flat buffers.
    p->n = A.elems;
    return JA_OK;
}

}  // namespace

// bf16 attention: 4 words of range-check flags per tile (fused tiles for
// ja_plan_run's workspace, per-tuple tiles after ja_kernel's partials)
static size_t att_flag_bytes(const ja_plan* p, int32_t ntiles) {
    return p->kind == JA_OP_ATTENTION && p->in_dtype == JA_BF16 ? (size_t)16 * (size_t)ntiles : 0;
}

extern "C" {

ja_status ja_plan_create(const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in, int32_t n_in,
                         const ja_relation_desc* out, ja_plan** plan) {
    if (!plan) return fail(JA_ERR_ARG, "plan is NULL");
    *plan = nullptr;
    if (!s || !d || !in || !out) return fail(JA_ERR_ARG, "NULL argument");
    if (d->letters != s->letters) return fail(JA_ERR_DECOMP, "decomposition was made for another spec");
    if (n_in != (int32_t)s->ins.size()) return fail(JA_ERR_ARG, "number of input relations differs from the spec");
    for (int i = 0; i < n_in; ++i)
        if (!in[i]) return fail(JA_ERR_ARG, "input relation descriptor is NULL");
    ja_tuples t;
    ja_status st = build_tuples(s, d, t);
    if (st) return st;
    ja_plan* p = new ja_plan();
    p->kind = s->kind;
    p->n_in = n_in;
    switch (s->kind) {
        case JA_OP_CONTRACT: st = plan_contract(p, s, d, t, in, out); break;
        case JA_OP_ATTENTION: st = plan_attention(p, s, d, t, in, out); break;
        case JA_OP_RMSNORM: st = plan_rmsnorm(p, s, d, in, out); break;
        default: st = plan_zip(p, s, d, in, out); break;
    }
    if (st) {
        delete p;
        return st;
    }
    if (p->table.empty()) p->table.resize(16, 0);
    *plan = p;
    return JA_OK;
}

ja_status ja_plan_device_bytes(const ja_plan* p, size_t* table_bytes, size_t* workspace_bytes) {
    if (!p) return fail(JA_ERR_ARG, "plan is NULL");
    if (table_bytes) *table_bytes = p->table.size();
    if (workspace_bytes) *workspace_bytes = att_flag_bytes(p, p->ntiles);
    return JA_OK;
}

ja_status ja_plan_upload(ja_plan* p, void* dev_buf, size_t bytes, void* stream) {
    if (!p || !dev_buf) return fail(JA_ERR_ARG, "NULL argument");
    if (bytes < p->table.size()) return fail(JA_ERR_WORKSPACE, "table buffer smaller than ja_plan_device_bytes");
    if ((uintptr_t)dev_buf & 15) return fail(JA_ERR_ARG, "table buffer must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    JA_TRY_HIP(hipMemcpyAsync(dev_buf, p->table.data(), p->table.size(), hipMemcpyHostToDevice, st));
    JA_TRY_HIP(hipStreamSynchronize(st));
    p->dev = dev_buf;
    return JA_OK;
}

static ja_status check_ptrs(const ja_plan* p, const void* const* in_ptrs, const void* out_ptr) {
    if (!p) return fail(JA_ERR_ARG, "plan is NULL");
    if (!p->dev) return fail(JA_ERR_STATE, "plan tables are not uploaded");
    if (!in_ptrs || !out_ptr) return fail(JA_ERR_ARG, "NULL buffer");
    for (int i = 0; i < p->n_in; ++i) {
        if (!in_ptrs[i]) return fail(JA_ERR_ARG, "NULL input buffer");
        if ((uintptr_t)in_ptrs[i] & 15) return fail(JA_ERR_ARG, "input buffers must be 16-byte aligned");
    }
    if ((uintptr_t)out_ptr & 15) return fail(JA_ERR_ARG, "output buffer must be 16-byte aligned");
    return JA_OK;
}

ja_status ja_plan_run(const ja_plan* p, const void* const* in_ptrs, void* out_ptr, void* workspace, void* stream) {
    ja_status st = check_ptrs(p, in_ptrs, out_ptr);
    if (st) return st;
    hipStream_t hs = (hipStream_t)stream;
    switch (p->kind) {
        case JA_OP_CONTRACT:
            if (p->ntiles == 0) return JA_OK;
            JA_TRY_HIP(launch_gemm(p->dev, p->tiles_off, p->ntiles, p->segs_off, p->tuples_off, in_ptrs[0], in_ptrs[1],
                                   out_ptr, p->epilogue == JA_EPI_ADD ? in_ptrs[2] : nullptr, p->epilogue,
                                   p->in_dtype, p->out_dtype, p->a_layout, p->b_layout, hs));
            break;
        case JA_OP_ATTENTION:
            if (p->ntiles == 0) return JA_OK;
            if (att_flag_bytes(p, p->ntiles) && !workspace)
                return fail(JA_ERR_WORKSPACE, "bf16 attention needs the plan's workspace");
            if ((uintptr_t)workspace & 15) return fail(JA_ERR_ARG, "workspace must be 16-byte aligned");
            JA_TRY_HIP(launch_attention(p->dev, p->tiles_off, p->ntiles, p->segs_off, p->tuples_off, p->seq_off,
                                        p->nseq, in_ptrs[0], in_ptrs[1], in_ptrs[2], out_ptr, (uint32_t*)workspace,
                                        p->scale, p->causal, p->in_dtype == JA_F16, 0, hs));
            break;
        case JA_OP_RMSNORM:
            JA_TRY_HIP(launch_rmsnorm(p->dev, p->rsplit_off, p->nrb, p->nblk_off, p->ndb, p->rows, p->D, p->norm_w,
                                      in_ptrs[0], in_ptrs[1], out_ptr, p->eps, p->norm_vec, p->in_dtype == JA_F16,
                                      hs));
            break;
        case JA_OP_SWIGLU:
            JA_TRY_HIP(launch_swiglu(in_ptrs[0], in_ptrs[1], out_ptr, p->n, p->in_dtype == JA_F16, hs));
            break;
        case JA_OP_ADD: JA_TRY_HIP(launch_add(in_ptrs[0], in_ptrs[1], out_ptr, p->n, p->in_dtype == JA_F16, hs)); break;
    }
    return JA_OK;
}

ja_status ja_plan_partial_bytes(const ja_plan* p, size_t* bytes) {
    if (!p || !bytes) return fail(JA_ERR_ARG, "NULL argument");
    if (p->kind != JA_OP_CONTRACT && p->kind != JA_OP_ATTENTION)
        return fail(JA_ERR_UNSUPPORTED, "unfused path exists for contract and attention only");
    if (p->epilogue != JA_EPI_NONE) return fail(JA_ERR_UNSUPPORTED, "unfused path exists for plain contractions only");
    if (p->att_inner) return fail(JA_ERR_UNSUPPORTED, INNER_UNFUSED);
    // bf16 attention: the per-tuple tiles' range-check flags follow the partials
    *bytes = (size_t)p->partial_elems * 4 + att_flag_bytes(p, p->nutiles);
    return JA_OK;
}

ja_status ja_kernel(const ja_plan* p, const void* const* in_ptrs, void* partials, void* stream) {
    ja_status st = check_ptrs(p, in_ptrs, partials);
    if (st) return st;
    if (p->kind != JA_OP_CONTRACT && p->kind != JA_OP_ATTENTION)
        return fail(JA_ERR_UNSUPPORTED, "unfused path exists for contract and attention only");
    if (p->epilogue != JA_EPI_NONE) return fail(JA_ERR_UNSUPPORTED, "unfused path exists for plain contractions only");
    if (p->att_inner) return fail(JA_ERR_UNSUPPORTED, INNER_UNFUSED);
    if (p->nutiles == 0) return JA_OK;
    hipStream_t hs = (hipStream_t)stream;
    if (p->kind == JA_OP_ATTENTION) {
        uint32_t* flags = (uint32_t*)((uint8_t*)partials + (size_t)p->partial_elems * 4);
        JA_TRY_HIP(launch_attention(p->dev, p->utiles_off, p->nutiles, p->usegs_off, p->tuples_off, p->seq_off,
                                    p->nseq, in_ptrs[0], in_ptrs[1], in_ptrs[2], partials, flags, p->scale,
                                    p->causal, p->in_dtype == JA_F16, 1, hs));
        return JA_OK;
    }
    JA_TRY_HIP(launch_gemm(p->dev, p->utiles_off, p->nutiles, p->usegs_off, p->tuples_off, in_ptrs[0], in_ptrs[1],
                           partials, nullptr, JA_EPI_NONE, p->in_dtype, JA_F32, p->a_layout, p->b_layout, hs));
    return JA_OK;
}

ja_status ja_agg(const ja_plan* p, ja_agg_op op, const void* partials, void* out_ptr, void* stream) {
    if (!p || !partials || !out_ptr) return fail(JA_ERR_ARG, "NULL argument");
    if (!p->dev) return fail(JA_ERR_STATE, "plan tables are not uploaded");
    if (p->kind != JA_OP_CONTRACT && p->kind != JA_OP_ATTENTION)
        return fail(JA_ERR_UNSUPPORTED, "unfused path exists for contract and attention only");
    if (p->epilogue != JA_EPI_NONE) return fail(JA_ERR_UNSUPPORTED, "unfused path exists for plain contractions only");
    if (p->att_inner) return fail(JA_ERR_UNSUPPORTED, INNER_UNFUSED);
    if (op != JA_AGG_SUM && op != JA_AGG_MAX && op != JA_AGG_SOFTMAX)
        return fail(JA_ERR_ARG, "unknown aggregation operator");
    if ((p->kind == JA_OP_ATTENTION) != (op == JA_AGG_SOFTMAX))
        return fail(JA_ERR_UNSUPPORTED, "attention partials aggregate with JA_AGG_SOFTMAX, contraction partials with "
                                        "JA_AGG_SUM or JA_AGG_MAX");
    if (((uintptr_t)partials & 15) || ((uintptr_t)out_ptr & 15)) return fail(JA_ERR_ARG, "buffers must be 16-byte aligned");
    if (p->natiles == 0) return JA_OK;
    if (op == JA_AGG_SOFTMAX) {
        JA_TRY_HIP(launch_smax_agg(p->dev, p->atiles_off, p->natiles, p->asegs_off, p->apoff_off,
                                   (const float*)partials, out_ptr, p->in_dtype == JA_F16, (hipStream_t)stream));
        return JA_OK;
    }
    JA_TRY_HIP(launch_agg(p->dev, p->atiles_off, p->natiles, p->asegs_off, p->apoff_off, (const float*)partials,
                          out_ptr, p->out_dtype, (int32_t)op, (hipStream_t)stream));
    return JA_OK;
}

void ja_plan_destroy(ja_plan* p) { delete p; }

ja_status ja_einsum_workspace_bytes(const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in,
                                    int32_t n_in, const ja_relation_desc* out, size_t* bytes) {
    if (!bytes) return fail(JA_ERR_ARG, "bytes is NULL");
    ja_plan* p = nullptr;
    ja_status st = ja_plan_create(s, d, in, n_in, out, &p);
    if (st) return st;
    size_t tb = 0, wb = 0;
    ja_plan_device_bytes(p, &tb, &wb);
    *bytes = ((tb + 255) & ~(size_t)255) + wb;
    ja_plan_destroy(p);
    return JA_OK;
}

ja_status ja_einsum(const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in,
                    const void* const* in_ptrs, int32_t n_in, const ja_relation_desc* out, void* out_ptr,
                    void* dev_ws, size_t ws_bytes, void* stream) {
    ja_plan* p = nullptr;
    ja_status st = ja_plan_create(s, d, in, n_in, out, &p);
    if (st) return st;
    size_t tb = 0, wb = 0;
    ja_plan_device_bytes(p, &tb, &wb);
    size_t tb_al = (tb + 255) & ~(size_t)255;
    if (!dev_ws || ws_bytes < tb_al + wb) {
        ja_plan_destroy(p);
        return fail(JA_ERR_WORKSPACE, "workspace smaller than ja_einsum_workspace_bytes");
    }
    st = ja_plan_upload(p, dev_ws, tb, stream);
    if (!st) st = ja_plan_run(p, in_ptrs, out_ptr, wb ? (char*)dev_ws + tb_al : nullptr, stream);
    ja_plan_destroy(p);
    return st;
}

}  // extern "C"
