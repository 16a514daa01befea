// dattn.cpp -- host side of the device-side attention planner: packed
// sequences whose ends are data on the GPU ("packed=device"), joined, planned
// and computed by kernels on one stream with no host round trip.
#include <cmath>
#include <cstring>

#include "../ja_dattn.h"
#include "ja_host.h"

namespace ja {
hipError_t launch_dattn_tables(const DAttnArgs& a, const int64_t* splits, const int32_t* rec, const int64_t* seg_off,
                               const int64_t* counts, const int64_t* qbase, const int32_t* qn, const int64_t* kbase,
                               const int32_t* kn, AttnSeg* segs, AttnTuple* tuples, AttnTile* tiles,
                               uint32_t* tcnt, uint32_t* hist, uint32_t* base, uint32_t* cursor, int32_t* ntiles,
                               int32_t* seq32, hipStream_t stream);
hipError_t launch_attention_dev(const AttnTile* tiles, const int32_t* ntiles_dev, uint32_t max_tiles,
                                const AttnSeg* segs, const AttnTuple* tuples, const int32_t* seq_ends, int32_t nseq,
                                const void* Q, const void* K, const void* V, void* O, uint32_t* flags, float scale,
                                int32_t causal, int32_t f16, hipStream_t stream);
namespace {
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per block of the given batch letters (lexicographic over their intervals):
// the batch-heads it holds and its first element ([block][bh][S][D] layout).
void blocks_of(const std::vector<int64_t>& ext, const std::vector<int32_t>& cnt, int64_t rowlen,
               std::vector<int64_t>& base, std::vector<int32_t>& n) {
    std::vector<std::vector<int64_t>> sp;
    int64_t nb = 1;
    for (size_t i = 0; i < ext.size(); ++i) {
        sp.push_back(equal_splits(ext[i], cnt[i]));
        nb *= cnt[i];
    }
    base.assign(nb, 0);
    n.assign(nb, 0);
    std::vector<int64_t> idx(ext.size(), 0);
    int64_t off = 0;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t r = b, bh = 1;
        for (int i = (int)ext.size() - 1; i >= 0; --i) {
            idx[i] = r % cnt[i];
            r /= cnt[i];
        }
        for (size_t i = 0; i < ext.size(); ++i) bh *= sp[i][idx[i] + 1] - sp[i][idx[i]];
        base[b] = off;
        n[b] = (int32_t)bh;
        off += bh * rowlen;
    }
}
}  // namespace
}  // namespace ja

struct ja_dattn {
    ja_djoin* dj = nullptr;
    ja::DAttnArgs a;
    std::vector<int64_t> qbase, kbase;
    std::vector<int32_t> qn, kn;
    size_t dj_table = 0, off_qbase = 0, off_qn = 0, off_kbase = 0, off_kn = 0, table_bytes = 0;
    size_t dj_ws = 0, off_rec = 0, off_seg = 0, off_tcnt = 0, off_hist = 0, off_base = 0, off_cursor = 0,
           off_ntiles = 0, off_segs = 0, off_tuples = 0, off_tiles = 0, off_seq = 0, off_flags = 0, ws_bytes = 0;
    int64_t n_splits = 0, max_tuples = 0, max_segs = 0;
    int32_t f16 = 0, causal = 0;
    float scale = 0;
    uint8_t* dev = nullptr;
};

using namespace ja;

extern "C" {

void ja_dattn_destroy(ja_dattn* d) {
    if (!d) return;
    ja_djoin_destroy(d->dj);
    delete d;
}

ja_status ja_dattn_create(const ja_spec* s, const int64_t* extents, const int32_t* intervals, int32_t dtype,
                          ja_dattn** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!s || !extents || !intervals) return fail(JA_ERR_ARG, "NULL argument");
    if (s->kind != JA_OP_ATTENTION || !s->packed_device)
        return fail(JA_ERR_SPEC, "the device planner takes attention with packed=device");
    if (dtype != JA_BF16 && dtype != JA_F16) return fail(JA_ERR_DTYPE, "attention relations are bf16 or f16");
    const std::string &q = s->ins[0], &k = s->ins[1];
    if (q[q.size() - 2] != s->att_s || k[k.size() - 2] != s->att_t)
        return fail(JA_ERR_UNSUPPORTED, "the device planner takes head-major relations (position letter second to last)");
    const int ls = s->letter_index(s->att_s), lt = s->letter_index(s->att_t);
    const int ld = s->letter_index(q.back());
    if (extents[ld] != ATTN_D) return fail(JA_ERR_UNSUPPORTED, "attention kernel is built for head dimension 128");
    if (extents[ls] > ((int64_t)1 << 31) - 1) return fail(JA_ERR_UNSUPPORTED, "sequence index beyond 2^31");
    ja_dattn* d = new ja_dattn();
    ja_status st = ja_djoin_create(s, extents, intervals, &d->dj);
    if (st) {
        delete d;
        return st;
    }
    DAttnArgs& a = d->a;
    std::memset(&a, 0, sizeof(a));
    a.nl = (int32_t)s->letters.size();
    a.ls = ls;
    a.lt = lt;
    a.D = ATTN_D;
    a.S = extents[ls];
    a.nseq = intervals[ls];
    std::vector<int64_t> qext, kext;
    std::vector<int32_t> qcnt, kcnt;
    int64_t total_bh = 1;
    for (size_t i = 0; i + 2 < q.size(); ++i) {
        const int l = s->letter_index(q[i]);
        a.qlet[a.nq] = l;
        a.qcnt[a.nq++] = intervals[l];
        qext.push_back(extents[l]);
        qcnt.push_back(intervals[l]);
        total_bh *= extents[l];
    }
    for (size_t i = 0; i + 2 < k.size(); ++i) {
        const int l = s->letter_index(k[i]);
        a.klet[a.nk] = l;
        a.kcnt[a.nk++] = intervals[l];
        kext.push_back(extents[l]);
        kcnt.push_back(intervals[l]);
    }
    int64_t sp_off = 0;
    for (int i = 0; i < a.nl; ++i) {
        if (i == ls) a.sp_s = (int32_t)sp_off;
        if (i == lt) a.sp_t = (int32_t)sp_off;
        sp_off += intervals[i] + 1;
    }
    blocks_of(qext, qcnt, a.S * a.D, d->qbase, d->qn);
    blocks_of(kext, kcnt, a.S * a.D, d->kbase, d->kn);
    size_t ws_dj = 0, tb_dj = 0;
    ja_djoin_device_bytes(d->dj, &tb_dj, &ws_dj, &d->max_tuples, &d->max_segs, &d->n_splits);
    const int64_t max_tiles = total_bh * ((a.S + ATTN_TQ - 1) / ATTN_TQ + a.nseq);
    if (max_tiles > ((int64_t)1 << 31) - 1 || d->max_segs > ((int64_t)1 << 31) - 1) {
        ja_dattn_destroy(d);
        return fail(JA_ERR_UNSUPPORTED, "more than 2^31 tiles");
    }
    a.max_segs = (uint32_t)d->max_segs;
    a.max_tuples = (uint32_t)d->max_tuples;
    a.max_tiles = (uint32_t)max_tiles;
    a.nbucket = (uint32_t)((a.S + ATTN_TQ - 1) / ATTN_TQ);
    d->f16 = dtype == JA_F16 ? 1 : 0;
    d->causal = s->causal ? 1 : 0;
    d->scale = (float)(s->has_scale ? s->scale : 1.0 / std::sqrt((double)ATTN_D));
    // device table: the join's table, then the batch-head block arrays
    size_t o = al256(tb_dj);
    d->dj_table = tb_dj;
    d->off_qbase = o;
    o = al256(o + 8 * d->qbase.size());
    d->off_qn = o;
    o = al256(o + 4 * d->qn.size());
    d->off_kbase = o;
    o = al256(o + 8 * d->kbase.size());
    d->off_kn = o;
    o = al256(o + 4 * d->kn.size());
    d->table_bytes = o;
    // workspace: the join's, its outputs, then the attention tables
    o = al256(ws_dj);
    d->dj_ws = ws_dj;
    d->off_rec = o;
    o = al256(o + 4 * (size_t)d->max_tuples * a.nl);
    d->off_seg = o;
    o = al256(o + 8 * ((size_t)d->max_segs + 1));
    d->off_tcnt = o;
    o = al256(o + 4 * (size_t)d->max_segs);
    d->off_hist = o;
    o = al256(o + 4 * (size_t)a.nbucket);
    d->off_base = o;
    o = al256(o + 4 * (size_t)a.nbucket);
    d->off_cursor = o;
    o = al256(o + 4 * (size_t)a.nbucket);
    d->off_ntiles = o;
    o = al256(o + 4);
    d->off_segs = o;
    o = al256(o + sizeof(AttnSeg) * (size_t)d->max_segs);
    d->off_tuples = o;
    o = al256(o + sizeof(AttnTuple) * (size_t)d->max_tuples);
    d->off_tiles = o;
    o = al256(o + sizeof(AttnTile) * (size_t)max_tiles);
    d->off_seq = o;
    o = al256(o + 4 * (size_t)a.nseq);
    // bf16: the attention tiles' range-check flags (4 words per tile)
    d->off_flags = o;
    if (!d->f16) o = al256(o + 16 * (size_t)max_tiles);
    d->ws_bytes = o;
    *out = d;
    return JA_OK;
}

ja_status ja_dattn_device_bytes(const ja_dattn* d, size_t* table_bytes, size_t* workspace_bytes, int64_t* n_splits) {
    if (!d) return fail(JA_ERR_ARG, "device planner is NULL");
    if (table_bytes) *table_bytes = d->table_bytes;
    if (workspace_bytes) *workspace_bytes = d->ws_bytes;
    if (n_splits) *n_splits = d->n_splits;
    return JA_OK;
}

ja_status ja_dattn_upload(ja_dattn* d, void* dev_buf, size_t bytes, void* stream) {
    if (!d || !dev_buf) return fail(JA_ERR_ARG, "NULL argument");
    if (bytes < d->table_bytes) return fail(JA_ERR_WORKSPACE, "table buffer smaller than ja_dattn_device_bytes");
    if ((uintptr_t)dev_buf & 255) return fail(JA_ERR_ARG, "table buffer must be 256-byte aligned");
    ja_status st = ja_djoin_upload(d->dj, dev_buf, d->dj_table, stream);
    if (st) return st;
    uint8_t* b = (uint8_t*)dev_buf;
    hipStream_t hs = (hipStream_t)stream;
    JA_TRY_HIP(hipMemcpyAsync(b + d->off_qbase, d->qbase.data(), 8 * d->qbase.size(), hipMemcpyHostToDevice, hs));
    JA_TRY_HIP(hipMemcpyAsync(b + d->off_qn, d->qn.data(), 4 * d->qn.size(), hipMemcpyHostToDevice, hs));
    JA_TRY_HIP(hipMemcpyAsync(b + d->off_kbase, d->kbase.data(), 8 * d->kbase.size(), hipMemcpyHostToDevice, hs));
    JA_TRY_HIP(hipMemcpyAsync(b + d->off_kn, d->kn.data(), 4 * d->kn.size(), hipMemcpyHostToDevice, hs));
    JA_TRY_HIP(hipStreamSynchronize(hs));
    d->dev = b;
    return JA_OK;
}

ja_status ja_dattn_run(const ja_dattn* d, const int64_t* splits_dev, const void* Q, const void* K, const void* V,
                       void* O, int64_t* counts, void* workspace, void* stream) {
    if (!d) return fail(JA_ERR_ARG, "device planner is NULL");
    if (!d->dev) return fail(JA_ERR_STATE, "device planner table is not uploaded");
    if (!splits_dev || !Q || !K || !V || !O || !counts || !workspace) return fail(JA_ERR_ARG, "NULL buffer");
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15)
        return fail(JA_ERR_ARG, "Q, K, V and O must be 16-byte aligned");
    if (((uintptr_t)splits_dev | (uintptr_t)counts) & 7) return fail(JA_ERR_ARG, "splits and counts must be 8-byte aligned");
    if ((uintptr_t)workspace & 255) return fail(JA_ERR_ARG, "workspace must be 256-byte aligned");
    uint8_t* ws = (uint8_t*)workspace;
    hipStream_t hs = (hipStream_t)stream;
    int32_t* rec = (int32_t*)(ws + d->off_rec);
    int64_t* seg = (int64_t*)(ws + d->off_seg);
    ja_status st = ja_djoin_run(d->dj, splits_dev, rec, seg, counts, ws, stream);
    if (st) return st;
    AttnSeg* segs = (AttnSeg*)(ws + d->off_segs);
    AttnTuple* tuples = (AttnTuple*)(ws + d->off_tuples);
    AttnTile* tiles = (AttnTile*)(ws + d->off_tiles);
    int32_t* ntiles = (int32_t*)(ws + d->off_ntiles);
    int32_t* seq32 = (int32_t*)(ws + d->off_seq);
    JA_TRY_HIP(launch_dattn_tables(d->a, splits_dev, rec, seg, counts, (const int64_t*)(d->dev + d->off_qbase),
                                   (const int32_t*)(d->dev + d->off_qn), (const int64_t*)(d->dev + d->off_kbase),
                                   (const int32_t*)(d->dev + d->off_kn), segs, tuples, tiles,
                                   (uint32_t*)(ws + d->off_tcnt), (uint32_t*)(ws + d->off_hist),
                                   (uint32_t*)(ws + d->off_base), (uint32_t*)(ws + d->off_cursor), ntiles, seq32, hs));
    JA_TRY_HIP(launch_attention_dev(tiles, ntiles, d->a.max_tiles, segs, tuples, seq32, d->a.nseq, Q, K, V, O,
                                    (uint32_t*)(ws + d->off_flags), d->scale, d->causal, d->f16, hs));
    return JA_OK;
}

}  // extern "C"
